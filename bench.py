#!/usr/bin/env python3
"""Benchmark of the causal linear-attention hot path on one MI355X.

One step = one pass over every stage of the path, each on its own batch of
synthetic inputs already resident in HBM:

  * chunked prefill (the headline): B=4, H=64, N=32768, d=128, block 128,
    bf16 q/k/v/o, fp32 state;
  * decode, fp32 state: 256 x 64 sequences, d=128, one token;
  * backward (gradients of the prefill) at the prefill's shape;
  * decode, bf16 state: the same, state stored in bf16; and with an OCP
    FP8 E4M3 state under per-sequence scales;
  * token-by-token prefill and chunked prefill at B=1, H=8, N=4096, d=128,
    block 64 (the crossover comparison), run after a 512 MiB cache flush.

The state buffers are in/out; each step continues from the state the
previous one left (a continuation of longer sequences), which changes no
work.  Every kernel is timed with HIP events on the stream it runs on;
`value` is the chunked prefill's throughput in tokens/s (B*N tokens, all
heads) over the timed steps.  Prints ONE JSON line.

``--only crossover`` sweeps the chunked and the token-by-token prefill over
N = 256 ... 32768 at the crossover shape (see crossover_sweep); the default
run includes the sweep at 5 launches a point (``crossover_sweep``).
``--only long`` times the long-context prefill (B=1, H=64, N=1048576, d=128,
block 128; 16 GiB per tensor) with the value-column split and with the
sequence split (see long_context).
``--only decode128`` times the decode workload's 128 consecutive steps,
launched one by one and replayed from a HIP graph (see decode_steps; the
default run includes it).
``--only ceiling`` measures the HBM bandwidth a plain streaming kernel
reaches for the path's read:write byte mixes (see hbm_stream_reference); the default
run includes it.
``--only drift`` measures the rounding drift of stored states against the
fp64 oracle along one 1M-token sequence (not part of a step; see
drift_report); the default run includes it with the oracle timings
(``drift``; left out with --no-cpu-baseline).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import itertools
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "prefill tokens/s + TFLOP/s (% bf16 MFMA peak); decode state GB/s (% HBM)"

PREFILL = dict(B=4, H=64, N=32768, d=128, block=128)
DECODE = dict(B=256, H=64, d=128)
SMALL = dict(B=1, H=8, N=4096, d=128, block=64)
# one GPU's share of the 1M-token sequence cut into 8 segments (sequence sharding)
SHARD = dict(B=1, H=64, N=131072, d=128, block=128)
SNAP_EVERY = 8  # blocks between prefix-cache state snapshots (every 1024 tokens)
DRAFTS = 4      # draft tokens verified per sequence in the speculative step

PREFILL_KERNEL_SOURCES = ["linear_attention_lightning_amd/csrc/prefill_bf16_kernel.hpp",
                          "linear_attention_lightning_amd/csrc/prefill_bf16.hip",
                          "linear_attention_lightning_amd/csrc/common.hpp",
                          "linear_attention_lightning_amd/csrc/kernels.hpp"]
PROBE_LIB = os.path.join(ROOT, "linear_attention_lightning_amd", "_lib", "libhbm_stream.so")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_bf16_B4_H64_N32768_d128_blk128_hbm_traffic.md")


def prefill_bytes(B, H, N, d, **_):
    """Algorithmic HBM bytes of one prefill: bf16 q, k, v read once and o
    written once (8 d bytes per token-head) plus the fp32 state read and
    written once per sequence (8 d^2 bytes)."""
    return B * H * (N * 8 * d + 8 * d * d)


def prefill_flops(B, H, N, d, block, **_):
    """Useful flop: 4 d^2 per token-head (state readout and update) plus the
    causal half of the intra-block product, 2 d (block + 1) per token-head."""
    return B * H * N * (4 * d * d + 2 * d * (block + 1))


def prefill_dense_flops(B, H, N, d, block, **_):
    """Flop as the matrix cores execute them (full masked tiles)."""
    return B * H * N * (4 * d * d + 4 * d * block)


def backward_bytes(B, H, N, d, **_):
    """Least HBM bytes of the gradients: bf16 q, k, v, dO read once and dq,
    dk, dv written once (14 d bytes per token-head), plus the fp32 gradient
    of S_0 written (4 d^2 per head; no S_0 and no final-state gradient)."""
    return B * H * (N * 14 * d + 4 * d * d)


def backward_design_bytes(B, H, N, d, **_):
    """Bytes the two launches move with the dV and dK passes fused (the
    default at this shape): the dQ pass reads dO, V, K and writes dq (8 d per
    token-head); the fused sweep reads K, V, Q, dO once and writes dk and dv
    (12 d); plus the fp32 gradient of S_0."""
    return B * H * (N * 20 * d + 4 * d * d)


def state_accumulate_bytes(B, H, N, d, **_):
    """bf16 k and v read once (4 d bytes per token-head) plus the fp32 state
    read and written once per sequence."""
    return B * H * (N * 4 * d + 8 * d * d)


def decode_bytes(B, H, d, state_bytes):
    """State read and written once plus q, k, v, o in bf16."""
    return B * H * (2 * d * d * state_bytes + 4 * d * 2)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or
    None when the summary is missing or was taken on other kernel sources."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel source hash:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"calibrated HBM bytes per launch:\s*`?([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(PREFILL_KERNEL_SOURCES):
        return None
    return float(m_bytes.group(1))


def _host(t):
    return t.float().cpu().numpy()


def _rel_err(a, b):
    import numpy as np
    den = float(np.max(np.abs(b)))
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / den) if den > 0 else float(np.max(np.abs(a)))


def cpu_baseline(prefill, small, decode, long_sample, reps: int = 3):
    """The fp64 oracle, timed on this host's cores on the values the GPU
    computed on (copied from device memory), and the GPU's outputs of the
    last timed step compared with it (max|gpu - oracle| / max|oracle|, for the
    outputs and the final states).  Times are medians of `reps` runs of the
    compute only (no copies, no generation):
      * the prefill workload (B=4 H=64 N=32768 d=128): batch entry 0, its 64
        heads -- the sample; the rate is reported in the metric's unit,
        tokens/s, one token being a position of all 64 heads;
      * the crossover workload (B=1 H=8 N=4096 d=128): all of it;
      * the decode workload (256 x 64 sequences, d=128): one step, all of it;
      * the long-context workload (B=1 H=64 N=2^20 d=128): the 4 heads of
        LONG_HEADS, one run; the whole-workload time is extrapolated (x16)
        and labelled so.
    prefill, small: (q, k, v, S_in, o, S_out) device tensors of the sampled
    heads; decode: (q, k, v, S_in, o, S_out) of the whole step; long_sample:
    from long_context(keep_sample=True), or None."""
    import numpy as np
    from oracle import oracle
    threads = oracle.default_threads()
    oracle.recurrence(np.zeros((1, 8, 16), np.float32), np.zeros((1, 8, 16), np.float32),
                      np.zeros((1, 8, 16), np.float32))  # load + warm the library

    def timed(fn):
        ts, out = [], None
        for _ in range(reps):
            t0 = time.perf_counter()
            out = fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2], out

    per_workload, errors = {}, {}
    # prefill and crossover workloads: the token-by-token fp64 recurrence
    for name, (tensors, H_all) in (("prefill_B4_H64_N32768", (prefill, 64)),
                                   ("crossover_B1_H8_N4096", (small, 8))):
        q, k, v, S_in, o_gpu, S_gpu = tensors
        qh, kh, vh = _host(q), _host(k), _host(v)
        S0 = S_in.double().cpu().numpy()
        dt, (o_ref, S_ref) = timed(lambda: oracle.recurrence(qh, kh, vh, S0, nthreads=threads))
        heads, N, d = qh.shape[-3], qh.shape[-2], qh.shape[-1]
        per_workload[name] = {"seconds_median": dt, "heads": heads, "tokens_per_head": N,
                         "head_tokens_per_s": heads * N / dt,
                         "tokens_per_s": heads * N / dt / H_all,
                         "gflops_fp64": heads * N * 4 * d * d / dt / 1e9}
        errors[name] = {"o": _rel_err(_host(o_gpu), o_ref), "state": _rel_err(S_gpu.cpu().numpy(), S_ref),
                        "heads_checked": heads}
    # decode workload: one step of all 16384 sequences from the state it started from
    q, k, v, S_in, o_gpu, S_gpu = decode
    qh, kh, vh = _host(q), _host(k), _host(v)
    S_start = S_in.double().cpu().numpy()
    state = {}

    def one_step():
        S = S_start.copy()
        o = oracle.decode_step(qh, kh, vh, S, nthreads=threads)
        state["S"] = S
        return o

    dt, o_ref = timed(one_step)
    nseq = qh.shape[0] * qh.shape[1]
    per_workload["decode_256x64_d128"] = {"seconds_median": dt, "sequences": nseq, "tokens_per_s": qh.shape[0] / dt,
                                     "state_GBps_fp64": nseq * 2 * 128 * 128 * 8 / dt / 1e9}
    errors["decode_256x64_d128"] = {"o": _rel_err(_host(o_gpu), o_ref),
                                    "state": _rel_err(S_gpu.cpu().numpy(), state["S"])}
    # long-context workload: 4 heads, one run
    if long_sample is not None:
        qh, kh, vh = long_sample["inputs"]
        t0 = time.perf_counter()
        o_ref, S_ref = oracle.recurrence(qh, kh, vh, nthreads=threads)
        dt = time.perf_counter() - t0
        N = qh.shape[-2]
        per_workload["long_B1_H64_N1048576"] = {
            "seconds_4_heads": dt, "heads": len(LONG_HEADS), "runs": 1,
            "extrapolated_seconds_64_heads": dt / -(-len(LONG_HEADS) // threads) * -(-64 // threads),
            "extrapolation": "extrapolated, not measured: the oracle runs one head per thread, so 64 heads take "
                             "ceil(64 / threads) rounds of the per-round time of the 4-head run",
            "head_tokens_per_s": len(LONG_HEADS) * N / dt}
        for way in ("seqsplit", "value_split"):
            o_gpu, S_gpu = long_sample[way]
            errors[f"long_B1_H64_N1048576_{way}"] = {"o": _rel_err(o_gpu, o_ref), "state": _rel_err(S_gpu, S_ref),
                                                     "heads_checked": list(LONG_HEADS)}
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((line.split(":", 1)[1].strip() for line in f if line.startswith("model name")), "")
    except OSError:
        pass
    head = per_workload["prefill_B4_H64_N32768"]
    baseline = {
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"prefill workload batch entry 0 (64 of the 256 sequences, N=32768, d=128), the GPU's own "
                  f"inputs and initial states, fp64 token-by-token recurrence, median of {reps} runs "
                  f"({head['seconds_median']:.2f} s each, {head['gflops_fp64']:.1f} GFLOP/s fp64)",
        "configs": per_workload,
    }
    return baseline, errors


LONG = dict(B=1, H=64, N=1 << 20, d=128, block=128)
DECODE_STEPS = 128  # consecutive single-token steps of the decode workload


def decode_steps(la, synth, torch, reps: int = 5):
    """The decode workload's 128 consecutive single-token steps (256 x 64
    sequences, d = 128, fp32 state from the 2048-outer-product S_0, fresh bf16
    q, k, v each step), timed as a whole: launched one by one, and captured
    once in a HIP graph and replayed.  The state is reset from S_0 outside
    the timed regions.  Every replay's outputs and final state are compared
    bitwise with the launched-one-by-one run (eager work and a
    synchronisation between replays)."""
    D = DECODE
    dev = torch.device("cuda:0")
    S0 = synth.decode_initial_state_device(D["B"], D["H"], D["d"])
    qs, ks, vs = (torch.stack(t) for t in zip(*(synth.decode_step_inputs_device(t, D["B"], D["H"], D["d"])
                                                  for t in range(DECODE_STEPS))))
    S = S0.clone()
    o = torch.empty_like(qs)

    def run():
        for t in range(DECODE_STEPS):
            la.decode(qs[t], ks[t], vs[t], o[t], S)

    def timed(fn):
        ms = []
        for _ in range(reps):
            S.copy_(S0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return sum(ms) / len(ms)

    eager_ms = timed(run)
    S_ref, o_ref = S.clone(), o.clone()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    S.copy_(S0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        run()
    torch.cuda.synchronize()
    same = True
    for _ in range(3):
        S.copy_(S0)
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = same and torch.equal(S, S_ref) and torch.equal(o, o_ref)
        # eager work between replays
        S.copy_(S0)
        run()
        torch.cuda.synchronize()
        same = same and torch.equal(S, S_ref)
    graph_ms = timed(graph.replay)
    # the same 128 steps with the state stored in bf16 (the precision hazard
    # of a low-precision stored state): error of its final state and of its
    # outputs against the fp32-state run
    S16 = S0.to(torch.bfloat16)
    o16 = torch.empty_like(o)
    for t in range(DECODE_STEPS):
        la.decode(qs[t], ks[t], vs[t], o16[t], S16)
    torch.cuda.synchronize()
    s_err = ((S16.float() - S_ref).abs().max() / S_ref.abs().max()).item()
    o_err = ((o16.float() - o_ref.float()).abs().max() / o_ref.float().abs().max()).item()
    step_bytes = decode_bytes(D["B"], D["H"], D["d"], 4)
    return {"steps": DECODE_STEPS,
            "eager_ms": eager_ms, "eager_ms_per_step": eager_ms / DECODE_STEPS,
            "graph_ms": graph_ms, "graph_ms_per_step": graph_ms / DECODE_STEPS,
            "graph_GBps": step_bytes * DECODE_STEPS / (graph_ms / 1e3) / 1e9,
            "graph_pct_hbm_peak": 100 * step_bytes * DECODE_STEPS / (graph_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "graph_replays_bitwise_equal_to_eager": bool(same),
            "bf16_state_vs_fp32_state_rel_err_after_128_steps": s_err,
            "bf16_state_outputs_vs_fp32_state_outputs_rel_err": o_err}


LONG_HEADS = (0, 21, 42, 63)  # heads of the long-context workload checked against the oracle


def long_context(la, synth, torch, steps: int = 5, keep_sample: bool = False):
    """The 1M-token prefill over 64 heads from a zero state, two ways:
    lin_attn_prefill (64 sequences; the value columns split 4 ways to fill
    the GPU) and lin_attn_prefill_seqsplit (each sequence cut into parts whose
    initial states come from the token-split K^T V of the parts before).  HIP
    events on the launch stream, `steps` timed launches after one untimed
    one; the state is reset outside the timed region.  With keep_sample, the
    inputs, outputs and final states of heads LONG_HEADS (batch entry 0) of
    the last launch of each way are returned as host arrays for the oracle
    leg."""
    L = LONG
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    q, k, v = synth.prefill_inputs_device(8, L["B"], L["H"], L["N"], L["d"])
    o = torch.empty_like(q)
    S = torch.zeros((L["B"], L["H"], L["d"], L["d"]), dtype=torch.float32, device=dev)
    ws_bytes = la.prefill_seqsplit_workspace(L["B"], L["H"], L["N"], L["d"], L["block"], torch.bfloat16)
    ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)
    hs = list(LONG_HEADS)
    res, sample = {}, {}
    for name, fn in (("value_split", lambda: la.prefill(q, k, v, o, S, L["block"])),
                     ("seqsplit", lambda: la.prefill_seqsplit(q, k, v, o, S, L["block"], ws))):
        ms = []
        for i in range(steps + 1):
            S.zero_()
            o.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if i > 0:
                ms.append(e0.elapsed_time(e1))
        res[name] = sorted(ms)[len(ms) // 2]
        if keep_sample:
            sample[name] = (o[0, hs].float().cpu().numpy(), S[0, hs].cpu().numpy())
    if keep_sample:
        sample["inputs"] = tuple(t[0, hs].float().cpu().numpy() for t in (q, k, v))
    del q, k, v, o, ws
    tokens = L["B"] * L["N"]
    nbytes = prefill_bytes(**L)
    B, H, N, d = L["B"], L["H"], L["N"], L["d"]
    out = {"metric": "long-context prefill time (ms per launch, median)",
           "config": {"workload": "B=1 H=64 N=1048576 d=128 block=128, bf16 q/k/v/o, fp32 state from zero"},
           "steps": steps, "algorithmic_bytes": nbytes, "seqsplit_workspace_bytes": ws_bytes}
    for name in ("seqsplit", "value_split"):
        t = res[name] / 1e3
        out[name] = {"ms": res[name], "tokens_per_s": tokens / t, "algorithmic_GBps": nbytes / t / 1e9,
                     "pct_hbm_peak": 100 * nbytes / t / 1e9 / PEAK_HBM_GBS,
                     "tflops_useful": prefill_flops(**L) / t / 1e12}
    # design bytes of the sequence split: the prefill's bytes plus K and V of
    # the first P-1 of the P parts read once more by the state pass, plus the
    # workspace states written and read once
    parts = seqsplit_parts(B * H, N)
    extra = B * H * N * 4 * d * (parts - 1) // parts + 2 * ws_bytes
    out["seqsplit"]["parts"] = parts
    out["seqsplit"]["design_bytes"] = nbytes + extra
    out["seqsplit"]["design_GBps"] = (nbytes + extra) / (res["seqsplit"] / 1e3) / 1e9
    out["value_split"]["design_note"] = ("each of the 4 value slices of a sequence reads all of q and k "
                                         "(its own quarter of v and o); the slices share an XCD's L2")
    return (out, sample) if keep_sample else out


def seqsplit_parts(BH: int, N: int, cus: int = 256) -> int:
    """Parts per sequence of lin_attn_prefill_seqsplit's plan (the library's
    own rule, restated for the byte model): the largest power of two P with
    B*H*P at most the compute-unit count, P dividing N and parts of at least
    512 tokens."""
    P = 1
    while BH * P * 2 <= cus and N % (P * 2) == 0 and N // (P * 2) >= 512:
        P *= 2
    return P


def hbm_stream_reference(torch, reps: int = 5):
    """HBM rates a plain streaming kernel reaches for each traffic mix of the
    path (csrc/hbm_stream.hip, its own library): 16-byte non-temporal loads,
    consecutive lanes at consecutive addresses.  A reference for the
    attention kernels' own mixes, not a bound on them (the decode step beats
    the 1:1 figure).  Measured for reads only, for 3 bytes read per byte
    written (the prefill's mix: q, k, v in, o out) and for 1:1, between two
    buffers and in place (the decode step reads and writes its state in
    place), each the best average over grid sizes and store policies, and
    over 1, 4 or 16 units loaded per wave before their stores.  The 3:1 mix is
    also measured with the prefill's own shape (hbm_stream_roles): one
    workgroup per compute unit, three waves each streaming one input, a
    fourth streaming the output.  HIP events on the launch stream, `reps`
    timed launches after 2 untimed ones."""
    lib = ctypes.CDLL(PROBE_LIB)
    lib.hbm_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hbm_stream_roles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    read_bytes = 6 << 30
    src = torch.ones(read_bytes // 4, dtype=torch.int32, device=dev)
    dst = torch.zeros(3 << 28, dtype=torch.int32, device=dev)  # 3 GiB
    unit = 4096

    def timed(fn, moved, name):
        ms = []
        for i in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"streaming probe {name} returned {rc}")
            if i >= 2:
                ms.append(e0.elapsed_time(e1))
        gbs = moved / (sum(ms) / len(ms) / 1e3) / 1e9
        if gbs > 1.05 * PEAK_HBM_GBS:  # the probe skipped work it was asked to do
            raise RuntimeError(f"streaming probe {name} measured {gbs:.0f} GB/s, above the HBM peak")
        return gbs

    mixes = {"read_only": (1, 0, read_bytes // unit, False), "r3w1": (3, 1, read_bytes // (3 * unit), False),
             "r1w1": (1, 1, (3 << 30) // unit, False),
             # in place: each 16-byte piece read and written back to the same
             # address, the access pattern of a state read-modify-write
             "r1w1_in_place": (1, 1, (3 << 30) // unit, True)}
    out = {}
    for name, (rd, wr, units, in_place) in mixes.items():
        moved = units * unit * (rd + wr)
        best = None
        for nt, wgs, batch in itertools.product((0, 1) if wr else (0,), (2048, 8192, 16384), (1, 4, 16)):
            target = src if in_place else dst
            gbs = timed(lambda: lib.hbm_stream(src.data_ptr(), target.data_ptr(), units, rd, wr, nt, wgs, batch,
                                               stream.cuda_stream), moved, name)
            if best is None or gbs > best[0]:
                best = (gbs, f"nt_store={nt} workgroups={wgs} batch={batch}")
        out[name + "_GBps"], out[name + "_config"] = best
    units = read_bytes // (3 * unit)
    best = None
    for nt, wgs, depth in itertools.product((0, 1), (256, 512), (8, 16)):
        gbs = timed(lambda: lib.hbm_stream_roles(src.data_ptr(), dst.data_ptr(), units, nt, wgs, depth,
                                                 stream.cuda_stream), units * unit * 4, "r3w1_roles")
        if best is None or gbs > best[0]:
            best = (gbs, f"nt_store={nt} workgroups={wgs} depth={depth}")
    out["r3w1_roles_GBps"], out["r3w1_roles_config"] = best
    del src, dst
    out["kernel"] = ("plain streaming kernels, 16-byte non-temporal loads, 256-lane workgroups "
                     "(csrc/hbm_stream.hip); r3w1_roles: three reading waves and one writing wave per workgroup")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg: its timing, the error check and the drift report")
    ap.add_argument("--only", choices=["prefill", "decode", "recurrent", "shard", "copy", "drift", "crossover",
                                       "ceiling", "long", "decode128"],
                    help="run one kernel only (for counter collection); prints timings, no JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path shards heads and sequences with no communication, "
              "and the measurement is of a single MI355X; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_lightning_amd as la
    from linear_attention_lightning_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    la.library()  # fail loudly before any setup if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only == "drift":
        print(json.dumps(drift_report(la, synth, torch)))
        return
    if args.only == "crossover":
        print(json.dumps(crossover_sweep(la, synth, torch, steps=args.steps)))
        return

    if args.only == "decode128":
        print(json.dumps(decode_steps(la, synth, torch)))
        return
    if args.only == "long":
        print(json.dumps(long_context(la, synth, torch)))
        return
    if args.only == "ceiling":
        print(json.dumps(hbm_stream_reference(torch)))
        return
    if args.only == "copy":
        # plain copy of a known size, used to calibrate the HBM byte counters
        n = 1 << 30
        x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        ms = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            y.copy_(x)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        avg_ms = sum(ms) / len(ms)
        print(f"copied {n} bytes x {args.steps}: avg {avg_ms:.4f} ms, {2 * n / (avg_ms / 1e3) / 1e9:.1f} GB/s "
              f"(read + write), best {2 * n / (min(ms) / 1e3) / 1e9:.1f} GB/s")
        return

    P, D, S = PREFILL, DECODE, SMALL
    need = {"prefill": args.only in (None, "prefill"), "decode": args.only in (None, "decode"),
            "small": args.only in (None, "recurrent"), "shard": args.only in (None, "shard")}
    SH = SHARD
    t_setup = time.time()
    if need["prefill"]:
        pq, pk, pv = synth.prefill_inputs_device(3, P["B"], P["H"], P["N"], P["d"])
        po = torch.empty_like(pq)
        pS = torch.zeros((P["B"], P["H"], P["d"], P["d"]), dtype=torch.float32, device=dev)
        # prefix-cache variant: a state snapshot every SNAP_EVERY blocks
        pS2 = torch.zeros_like(pS)
        psnap = torch.empty((P["B"], P["H"], la.snapshot_count(P["N"], P["block"], SNAP_EVERY), P["d"], P["d"]),
                            dtype=torch.float32, device=dev)
        # backward: upstream gradients of the outputs, gradients written
        pdo = synth.prefill_inputs_device(5, P["B"], P["H"], P["N"], P["d"])[2]
        pdq, pdk, pdv = (torch.empty_like(pq) for _ in range(3))
        pdS0 = torch.empty_like(pS)
    if need["decode"]:
        dS32 = synth.decode_initial_state_device(D["B"], D["H"], D["d"])
        dS16 = dS32.to(torch.bfloat16)
        # E4M3 state under per-sequence power-of-two scales (largest stored
        # magnitude between 112 and 224, below the format's 448)
        dscale = torch.exp2(torch.ceil(torch.log2(dS32.abs().amax(dim=(2, 3)) / 224.0)))
        dS8 = (dS32 / dscale[:, :, None, None]).to(torch.float8_e4m3fn)
        dq, dk, dv = synth.decode_step_inputs_device(0, D["B"], D["H"], D["d"])
        do = torch.empty_like(dq)
        # speculative step: DRAFTS drafts per sequence, verified then committed
        # with per-sequence accepted counts (here: all but the last draft)
        tq, tk, tv = synth.prefill_inputs_device(7, D["B"], D["H"], DRAFTS, D["d"])
        to = torch.empty_like(tq)
        tacc = torch.full((D["B"],), DRAFTS - 1, dtype=torch.int32, device=dev)
    if need["small"]:
        sq, sk, sv = synth.prefill_inputs_device(2, S["B"], S["H"], S["N"], S["d"])
        so = torch.empty_like(sq)
        sS = torch.zeros((S["B"], S["H"], S["d"], S["d"]), dtype=torch.float32, device=dev)
        so2 = torch.empty_like(sq)
        sS2 = torch.zeros_like(sS)
        so3 = torch.empty_like(sq)
        sS3 = torch.zeros_like(sS)
        sws = torch.empty(max(16, la.prefill_seqsplit_workspace(S["B"], S["H"], S["N"], S["d"], S["block"],
                                                                torch.bfloat16)), dtype=torch.uint8, device=dev)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    if need["shard"]:
        hq, hk, hv = synth.prefill_inputs_device(4, SH["B"], SH["H"], SH["N"], SH["d"])
        ho = torch.empty_like(hq)
        # a non-zero initial state: the prefix sum of the earlier segments
        hS0 = torch.zeros((SH["B"], SH["H"], SH["d"], SH["d"]), dtype=torch.float32, device=dev)
        la.state_accumulate(hk, hv, hS0)
        hdS = torch.zeros_like(hS0)
        hdS2 = torch.zeros_like(hS0)
        hS0b = hS0.clone()
        ho2 = torch.empty_like(hq)
        hpws = torch.empty(max(16, la.prefill_seqsplit_workspace(SH["B"], SH["H"], SH["N"], SH["d"], SH["block"],
                                                                 torch.bfloat16)),
                           dtype=torch.uint8, device=dev)
        hws = torch.empty(max(16, la.state_accumulate_split_workspace(SH["B"], SH["H"], SH["N"], SH["d"],
                                                                      torch.bfloat16)),
                          dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    names = [n for n, on in (("prefill", need["prefill"]), ("prefill_snapshots", need["prefill"]),
                             ("backward", need["prefill"]),
                             ("decode_fp32", need["decode"]),
                             ("decode_bf16", need["decode"]), ("decode_e4m3", need["decode"]),
                             ("verify", need["decode"]),
                             ("commit", need["decode"]), ("small_chunked", need["small"]),
                             ("small_chunked_seqsplit", need["small"]),
                             ("small_recurrent", need["small"]), ("shard_state_accumulate", need["shard"]),
                             ("shard_state_accumulate_tiles", need["shard"]),
                             ("shard_prefill_seqsplit", need["shard"]),
                             ("shard_prefill", need["shard"])) if on]

    # The states are in/out and carry over from step to step; before the last
    # timed step each is copied (outside every kernel's event pair) so that
    # the oracle leg can check that step's outputs from the state they started
    # from.
    last_in = {}

    def keep(name, t):
        last_in[name] = t.clone()

    def step(evs, last=False):
        def timed(name, fn):
            if evs is not None:
                evs[name][0].record(stream)
            fn()
            if evs is not None:
                evs[name][1].record(stream)
        if need["prefill"]:
            if last:
                last_in["prefill_S"] = pS[0].clone()  # batch entry 0: the oracle leg's sample
            timed("prefill", lambda: la.prefill(pq, pk, pv, po, pS, P["block"]))
            if last:
                last_in["prefill_o"] = po[0].clone()
                last_in["prefill_SN"] = pS[0].clone()
            timed("prefill_snapshots", lambda: la.prefill_snapshots(pq, pk, pv, po, pS2, psnap, P["block"],
                                                                    SNAP_EVERY))
            timed("backward", lambda: la.backward(pq, pk, pv, pdo, pdq, pdk, pdv, P["block"], dstate0=pdS0))
        # The shard's kernels run right after the 32K-token passes, and the
        # decode group after them: the speculative verify, a read-only pass
        # over 1 GiB of states, measured 15 % slower (same clock, same
        # requests, a higher L2 read latency) whenever the decode group
        # followed the 32K-token passes or the crossover trio, and not after
        # the shard's kernels or at the start of a step.
        if need["shard"]:
            timed("shard_state_accumulate", lambda: la.state_accumulate_split(hk, hv, hdS, hws))
            timed("shard_state_accumulate_tiles", lambda: la.state_accumulate(hk, hv, hdS2))
            timed("shard_prefill", lambda: la.prefill(hq, hk, hv, ho, hS0, SH["block"]))
            timed("shard_prefill_seqsplit", lambda: la.prefill_seqsplit(hq, hk, hv, ho2, hS0b, SH["block"], hpws))
        if need["decode"]:
            if last:
                keep("decode_S", dS32)
            timed("decode_fp32", lambda: la.decode(dq, dk, dv, do, dS32))
            if last:
                keep("decode_o", do)
                keep("decode_SN", dS32)
            timed("decode_bf16", lambda: la.decode(dq, dk, dv, do, dS16))
            timed("decode_e4m3", lambda: la.decode(dq, dk, dv, do, dS8, state_scale=dscale))
            timed("verify", lambda: la.decode_verify(tq, tk, tv, to, dS32))
            timed("commit", lambda: la.decode_commit(tk, tv, dS32, tacc))
        if need["small"]:
            flush.fill_(0)
            if last:
                keep("small_S", sS)
            timed("small_chunked", lambda: la.prefill(sq, sk, sv, so, sS, S["block"]))
            if last:
                keep("small_o", so)
                keep("small_SN", sS)
            flush.fill_(1)
            timed("small_recurrent", lambda: la.prefill_recurrent(sq, sk, sv, so2, sS2))
            flush.fill_(0)
            timed("small_chunked_seqsplit", lambda: la.prefill_seqsplit(sq, sk, sv, so3, sS3, S["block"], sws))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    evs_all = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        evs = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
        step(evs, last=(i == args.steps - 1))
        evs_all.append(evs)
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    total_ms = start.elapsed_time(end)
    kern_ms = {n: [e[n][0].elapsed_time(e[n][1]) for e in evs_all] for n in names}
    avg = {n: sum(v) / len(v) for n, v in kern_ms.items()}
    best = {n: min(v) for n, v in kern_ms.items()}

    if args.only:
        for n in names:
            print(f"{n}: avg {avg[n]:.4f} ms, min {best[n]:.4f} ms over {args.steps} launches")
        return

    ceiling = hbm_stream_reference(torch)
    steps128 = decode_steps(la, synth, torch)
    # drop the shard's and the backward's buffers before the 64 GiB long-context inputs
    if need["shard"]:
        del hq, hk, hv, ho, ho2, hS0, hS0b, hdS, hdS2, hws, hpws
    if need["prefill"]:
        del pdo, pdq, pdk, pdv
    torch.cuda.empty_cache()
    long_res = long_context(la, synth, torch, keep_sample=not args.no_cpu_baseline)
    long_res, long_sample = long_res if isinstance(long_res, tuple) else (long_res, None)
    # the crossover sweep over sequence length (8 and 256 heads), 5 launches a point
    sweep = crossover_sweep(la, synth, torch, steps=5)
    p_bytes = prefill_bytes(**P)
    p_flops = prefill_flops(**P)
    p_dense = prefill_dense_flops(**P)
    p_s = avg["prefill"] / 1e3
    tokens = P["B"] * P["N"]
    gbs = p_bytes / p_s / 1e9
    traffic = measured_traffic()
    d32_bytes = decode_bytes(D["B"], D["H"], D["d"], 4)
    d16_bytes = decode_bytes(D["B"], D["H"], D["d"], 2)
    d8_bytes = decode_bytes(D["B"], D["H"], D["d"], 1)
    small_tokens = S["B"] * S["N"]

    out = {
        "metric": METRIC,
        "value": tokens / p_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal linear attention prefill, phi = identity, B=4 H=64 N=32768 d=128 block=128, "
                        "bf16 q/k/v/o, fp32 state",
            "decode_workload": "256 x 64 sequences, d=128, one token per step, fp32, bf16 and E4M3 states",
            "crossover_workload": "B=1 H=8 N=4096 d=128 block=64: chunked vs token-by-token",
        },
        "prefill": {
            "ms": avg["prefill"], "ms_min": best["prefill"],
            "ms_median": sorted(kern_ms["prefill"])[len(kern_ms["prefill"]) // 2],
            "tokens_per_s": tokens / p_s,
            "tflops_useful": p_flops / p_s / 1e12,
            "tflops_dense_tile": p_dense / p_s / 1e12,
            "pct_bf16_mfma_peak_useful": 100 * p_flops / p_s / 1e12 / PEAK_BF16_TFLOPS,
            "pct_bf16_mfma_peak_dense_tile": 100 * p_dense / p_s / 1e12 / PEAK_BF16_TFLOPS,
            "mfma_pct_ceiling_at_hbm_peak_useful": 100 * p_flops / (p_bytes / (PEAK_HBM_GBS * 1e9)) / 1e12
            / PEAK_BF16_TFLOPS,
            "hbm_GBps": gbs, "pct_hbm_peak": 100 * gbs / PEAK_HBM_GBS,
            "hbm_floor_ms": p_bytes / (PEAK_HBM_GBS * 1e9) * 1e3,
            "with_snapshots_ms": avg["prefill_snapshots"],
            "snapshot_every_tokens": SNAP_EVERY * P["block"],
            "snapshot_bytes": psnap.numel() * 4,
        },
        "backward": {
            "ms": avg["backward"],
            "tokens_per_s": tokens / (avg["backward"] / 1e3),
            "minimal_bytes": backward_bytes(**P),
            "hbm_GBps_minimal_bytes": backward_bytes(**P) / (avg["backward"] / 1e3) / 1e9,
            "design_bytes": backward_design_bytes(**P),
            "hbm_GBps_design_bytes": backward_design_bytes(**P) / (avg["backward"] / 1e3) / 1e9,
            "pct_hbm_peak_design_bytes": 100 * backward_design_bytes(**P) / (avg["backward"] / 1e3) / 1e9
            / PEAK_HBM_GBS,
            "launches": 2,
        },
        "decode": {
            "fp32_state_ms": avg["decode_fp32"], "fp32_state_GBps": d32_bytes / (avg["decode_fp32"] / 1e3) / 1e9,
            "fp32_state_pct_hbm_peak": 100 * d32_bytes / (avg["decode_fp32"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "bf16_state_ms": avg["decode_bf16"], "bf16_state_GBps": d16_bytes / (avg["decode_bf16"] / 1e3) / 1e9,
            "bf16_state_pct_hbm_peak": 100 * d16_bytes / (avg["decode_bf16"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "e4m3_state_ms": avg["decode_e4m3"], "e4m3_state_GBps": d8_bytes / (avg["decode_e4m3"] / 1e3) / 1e9,
            "e4m3_state_pct_hbm_peak": 100 * d8_bytes / (avg["decode_e4m3"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "tokens_per_s_fp32_state": D["B"] / (avg["decode_fp32"] / 1e3),
            "fp32_state_pct_of_1to1_stream_reference": 100 * d32_bytes / (avg["decode_fp32"] / 1e3) / 1e9
            / ceiling["r1w1_GBps"],
            "fp32_state_pct_of_in_place_1to1_stream_reference": 100 * d32_bytes / (avg["decode_fp32"] / 1e3) / 1e9
            / ceiling["r1w1_in_place_GBps"],
            "steps_128": steps128,
            "speculative": {
                "drafts": DRAFTS, "accepted": DRAFTS - 1,
                "verify_ms": avg["verify"], "commit_ms": avg["commit"],
                "verify_state_GBps": D["B"] * D["H"] * D["d"] ** 2 * 4 / (avg["verify"] / 1e3) / 1e9,
                "commit_state_GBps": 2 * D["B"] * D["H"] * D["d"] ** 2 * 4 / (avg["commit"] / 1e3) / 1e9,
                "vs_decode_steps": DRAFTS * avg["decode_fp32"] / (avg["verify"] + avg["commit"]),
            },
        },
        "crossover": {
            "chunked_ms": avg["small_chunked"], "recurrent_ms": avg["small_recurrent"],
            "chunked_seqsplit_ms": avg["small_chunked_seqsplit"],
            "chunked_seqsplit_ms_median": sorted(kern_ms["small_chunked_seqsplit"])[len(kern_ms["small_chunked_seqsplit"]) // 2],
            "chunked_seqsplit_ms_min": best["small_chunked_seqsplit"],
            "recurrent_ms_median": sorted(kern_ms["small_recurrent"])[len(kern_ms["small_recurrent"]) // 2],
            "chunked_seqsplit_tokens_per_s": small_tokens / (avg["small_chunked_seqsplit"] / 1e3),
            "chunked_tokens_per_s": small_tokens / (avg["small_chunked"] / 1e3),
            "recurrent_tokens_per_s": small_tokens / (avg["small_recurrent"] / 1e3),
            "cache": "each run follows a 512 MiB write that evicts the 256 MB last-level cache",
        },
        "sequence_shard": {
            "workload": "one of 8 segments of the 1M-token sequence: B=1 H=64 N=131072 d=128, bf16",
            "state_accumulate_ms": avg["shard_state_accumulate"],
            "state_accumulate_GBps": state_accumulate_bytes(**SH) / (avg["shard_state_accumulate"] / 1e3) / 1e9,
            "state_accumulate_kernel": "token-split (lin_attn_state_accumulate_split): one workgroup per "
                                       "(sequence, chunk), chunk sums added in order",
            "state_accumulate_tiles_ms": avg["shard_state_accumulate_tiles"],
            "state_accumulate_tiles_GBps": state_accumulate_bytes(**SH)
            / (avg["shard_state_accumulate_tiles"] / 1e3) / 1e9,
            "state_accumulate_pct_of_read_only_stream_reference": 100 * state_accumulate_bytes(**SH)
            / (avg["shard_state_accumulate"] / 1e3) / 1e9 / ceiling["read_only_GBps"],
            "prefill_nonzero_S0_ms": avg["shard_prefill"],
            "prefill_nonzero_S0_GBps": prefill_bytes(**SH) / (avg["shard_prefill"] / 1e3) / 1e9,
            "prefill_nonzero_S0_kernel": "lin_attn_prefill: 64 sequences, value columns split 4 ways",
            "prefill_seqsplit_nonzero_S0_ms": avg["shard_prefill_seqsplit"],
            "prefill_seqsplit_nonzero_S0_tokens_per_s": SH["B"] * SH["N"] / (avg["shard_prefill_seqsplit"] / 1e3),
            "prefill_seqsplit_algorithmic_GBps": prefill_bytes(**SH) / (avg["shard_prefill_seqsplit"] / 1e3) / 1e9,
            "prefill_seqsplit_kernel": "lin_attn_prefill_seqsplit: 4 parts per sequence, part states from the "
                                       "token-split K^T V of the parts before, 256 part prefills",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "prefill_bf16_kernel<128,128>",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes": p_bytes,
            # the best rate a plain streaming kernel reaches for the same 3:1
            # read:write mix on this GPU (hbm_stream_reference): context, not
            # a bound (8 TB/s is the peak frac is taken against)
            "same_mix_stream_reference_GBps": max(ceiling["r3w1_GBps"], ceiling["r3w1_roles_GBps"]),
            "frac_of_same_mix_stream_reference": gbs / max(ceiling["r3w1_GBps"], ceiling["r3w1_roles_GBps"]),
        },
        "long": long_res,
        "crossover_sweep": sweep,
        "hbm_stream_reference": ceiling,
        "timing": {"wall_ms_timed_region": wall_ms, "setup_s": setup_s,
                   "method": "HIP events on the launch stream around each kernel"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["error_vs_oracle"] = cpu_baseline(
            (pq[0], pk[0], pv[0], last_in["prefill_S"], last_in["prefill_o"], last_in["prefill_SN"]),
            (sq, sk, sv, last_in["small_S"], last_in["small_o"], last_in["small_SN"]),
            (dq, dk, dv, last_in["decode_S"], last_in["decode_o"], last_in["decode_SN"]),
            long_sample)
        out["error_vs_oracle"]["gates"] = {"bf16_io_fp32_state": 1e-2, "fp32_io": 1e-4}
        # the oracle leg also gives the stored-state drift along one 1M-token
        # sequence (about 25 s, with its own progress lines on stderr)
        out["drift"] = drift_report(la, synth, torch)
    print(json.dumps(out))



CROSSOVER = dict(B=1, Hs=(8, 256), d=128, block=64, Ns=(256, 512, 1024, 2048, 4096, 8192, 16384, 32768))


def crossover_sweep(la, synth, torch, steps: int = 20):
    """Chunked ("Lightning") prefill against the token-by-token recurrence
    over sequence length, at B=1 d=128 block 64 with 8 heads (the crossover
    shape; its 32 workgroups leave most of the GPU idle) and with 256 heads
    (a full GPU): where does the tiled form start to pay ("ノーフリーランチ"
    (winzheng.jp), section "計算とメモリのボトルネックの不整合": a
    break-even of a few thousand tokens)?  Each launch follows a 512 MiB
    write that evicts the last-level cache; times are HIP-event averages
    over `steps` launches.  The chunked form runs as lin_attn_prefill and as
    lin_attn_prefill_seqsplit (which cuts the sequences into parts of at
    least 256 tokens to fill the GPU).  A modeled line gives causal softmax attention at
    the bf16 matrix peak, 2 N^2 d flop per head (not built; context only).
    """
    B, d, blk = CROSSOVER["B"], CROSSOVER["d"], CROSSOVER["block"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    rows = []
    for H, N in ((H, N) for H in CROSSOVER["Hs"] for N in CROSSOVER["Ns"]):
        q, k, v = synth.prefill_inputs_device(12, B, H, N, d)
        o = torch.empty_like(q)
        S = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
        res = {}
        ws = torch.empty(max(16, la.prefill_seqsplit_workspace(B, H, N, d, blk, torch.bfloat16)),
                         dtype=torch.uint8, device=dev)
        for name, fn in (("chunked", lambda: la.prefill(q, k, v, o, S, blk)),
                         ("chunked_seqsplit", lambda: la.prefill_seqsplit(q, k, v, o, S, blk, ws)),
                         ("recurrent", lambda: la.prefill_recurrent(q, k, v, o, S))):
            ms = []
            for i in range(steps + 2):
                flush.fill_(i & 1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                if i >= 2:
                    ms.append(e0.elapsed_time(e1))
            res[name] = sum(ms) / len(ms)
        softmax_ms = 2.0 * N * N * d * B * H / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        rows.append({"H": H, "N": N, "chunked_ms": res["chunked"], "recurrent_ms": res["recurrent"],
                     "chunked_seqsplit_ms": res["chunked_seqsplit"],
                     "recurrent_over_chunked": res["recurrent"] / res["chunked"],
                     "chunked_tokens_per_s": B * N / (res["chunked"] / 1e3),
                     "recurrent_tokens_per_s": B * N / (res["recurrent"] / 1e3),
                     "modeled_softmax_at_bf16_peak_ms": softmax_ms})
        print(f"[crossover] H={H} N={N}: chunked {res['chunked']:.4f} ms, seqsplit {res['chunked_seqsplit']:.4f} ms, "
              f"recurrent {res['recurrent']:.4f} ms",
              file=sys.stderr, flush=True)
    return {"metric": "chunked vs token-by-token prefill time over N (ms per launch)",
            "config": {"workload": f"B={B} H in {list(CROSSOVER['Hs'])} d={d} block {blk}, "
                                   "bf16 q/k/v/o, fp32 state, cold cache"},
            "data": "synthetic", "steps": steps, "rows": rows}


DRIFT = dict(H=4, d=128, block=128, checkpoints=(1024, 4096, 16384, 65536, 262144, 1048576))


def drift_report(la, synth, torch):
    """Rounding drift of a stored state along one sequence, against the fp64
    oracle (the hazard of low-precision state storage: "ノーフリーランチ"
    (winzheng.jp), section "推論システム統合の課題").

    One sequence of 2^20 tokens (B=1, H=4, d=128; the synthetic recipe:
    q, k ~ N(0, 1/d), v ~ N(0, 1), bf16) is processed by
      * decode, one token per launch, with the state stored in fp32, bf16
        and E4M3 after every token;
      * chunked prefill (block 128) with an fp32 carry, and with the carry
        stored in bf16 or E4M3 after every block (lin_attn_prefill_scaled,
        round_carry = 1);
      * chunked prefill that stores bf16 / E4M3 once, at the end
        (round_carry = 0): one rounding, the floor of each format.
    E4M3 states use one power-of-two scale per head, fixed for the whole
    sequence: the smallest that maps the largest exact |S| over the sequence
    to at most 224.  At each checkpoint N the stored state is compared with
    the exact S_N (oracle.state_after, fp64) and the output of token N-1
    with the oracle's recurrence: relative errors max|x - x_exact| /
    max|x_exact|."""
    import numpy as np
    from oracle import oracle

    H, d, blk, cps = DRIFT["H"], DRIFT["d"], DRIFT["block"], DRIFT["checkpoints"]
    Nmax = cps[-1]
    t0 = time.time()
    q, k, v = synth.prefill_inputs_device(11, 1, H, Nmax, d)
    kh = k.float().cpu().numpy()
    vh = v.float().cpu().numpy()
    # exact states at every checkpoint (and one block before it)
    S_pre, S_cp = {}, {}
    S = np.zeros((1, H, d, d))
    last = 0
    for N in cps:
        S_pre[N] = oracle.state_after(kh[:, :, last:N - blk], vh[:, :, last:N - blk], S)
        S = oracle.state_after(kh[:, :, N - blk:N], vh[:, :, N - blk:N], S_pre[N])
        S_cp[N] = S
        last = N
    smax = max(float(np.abs(S_cp[N]).max()) for N in cps)
    head_max = np.max(np.stack([np.abs(S_cp[N]).max(axis=(2, 3)) for N in cps]), axis=0)  # [1, H]
    scale = np.exp2(np.ceil(np.log2(head_max / 224.0))).astype(np.float32)
    o_ref = {}
    for N in cps:
        qb = q[:, :, N - blk:N].float().cpu().numpy()
        o_ref[N] = oracle.recurrence(qb, kh[:, :, N - blk:N], vh[:, :, N - blk:N], S_pre[N])[0][:, :, -1]
    print(f"[drift] exact states ready ({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)

    dev = q.device
    scd = torch.from_numpy(scale).to(dev)
    fmts = {"bf16": (torch.bfloat16, oracle.FMT_BF16), "e4m3": (torch.float8_e4m3fn, oracle.FMT_E4M3)}

    def widen(t, fmt):
        if fmt == "fp32":
            return t.double().cpu().numpy()
        codes = t.cpu().view(torch.int16 if fmt == "bf16" else torch.uint8).numpy()
        if fmt == "bf16":
            codes = codes.view(np.uint16)
        return oracle.stored_to_f64(codes, fmts[fmt][1], scale if fmt == "e4m3" else None)

    def err(x, ref):
        return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))

    rows = {N: {"N": N, "state": {}, "output": {}} for N in cps}
    o = torch.empty_like(q)
    # chunked prefill, chained over the checkpoints (a continuation; with the
    # carry rounded every block this is the same computation as one call)
    for name, fmt, rc in (("prefill_fp32_carry", "fp32", None), ("prefill_bf16_carry", "bf16", True),
                          ("prefill_e4m3_carry", "e4m3", True)):
        st = torch.zeros((1, H, d, d), dtype=torch.float32, device=dev)
        if fmt != "fp32":
            st = st.to(fmts[fmt][0])
        last = 0
        for N in cps:
            sl = slice(last, N)
            seg = [t[:, :, sl].contiguous() for t in (q, k, v)]
            os_ = torch.empty_like(seg[0])
            if fmt == "fp32":
                la.prefill(*seg, os_, st, blk)
            else:
                la.prefill_scaled(*seg, os_, st, blk, state_scale=scd if fmt == "e4m3" else None, round_carry=rc)
            torch.cuda.synchronize()
            rows[N]["state"][name] = err(widen(st, fmt), S_cp[N])
            rows[N]["output"][name] = err(os_[:, :, -1].float().cpu().numpy(), o_ref[N])
            last = N
    # one rounding at the end
    for name, fmt in (("prefill_bf16_once", "bf16"), ("prefill_e4m3_once", "e4m3")):
        for N in cps:
            st = torch.zeros((1, H, d, d), dtype=fmts[fmt][0], device=dev)
            la.prefill_scaled(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(),
                              o[:, :, :N].contiguous(), st, blk, state_scale=scd if fmt == "e4m3" else None,
                              round_carry=False)
            torch.cuda.synchronize()
            rows[N]["state"][name] = err(widen(st, fmt), S_cp[N])
    print(f"[drift] prefill paths done ({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)
    # decode: token-major copies so each token's [1, H, d] slice is contiguous;
    # the C entry points are called directly with per-token pointers
    qt, kt, vt = (t.permute(2, 0, 1, 3).contiguous() for t in (q, k, v))
    lib = la.library()
    step = H * d * 2
    states = {"fp32": torch.zeros((1, H, d, d), dtype=torch.float32, device=dev),
              "bf16": torch.zeros((1, H, d, d), dtype=torch.bfloat16, device=dev),
              "e4m3": torch.zeros((1, H, d, d), dtype=torch.float8_e4m3fn, device=dev)}
    outs = {f: torch.empty((1, H, d), dtype=torch.bfloat16, device=dev) for f in states}
    code = {"fp32": la.F32, "bf16": la.BF16, "e4m3": la.FP8_E4M3}
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    qp, kp, vp = qt.data_ptr(), kt.data_ptr(), vt.data_ptr()
    sp = {f: states[f].data_ptr() for f in states}
    op = {f: outs[f].data_ptr() for f in states}
    scp = scd.data_ptr()
    t_done = 0
    for N in cps:
        for t in range(t_done, N):
            off = t * step
            for f in ("fp32", "bf16", "e4m3"):
                rc = lib.lin_attn_decode_scaled(qp + off, kp + off, vp + off, op[f], sp[f], scp, 1, H, d, la.BF16,
                                                code[f], stream) if f == "e4m3" else \
                    lib.lin_attn_decode(qp + off, kp + off, vp + off, op[f], sp[f], 1, H, d, la.BF16, code[f], stream)
                if rc != 0:
                    raise la.LinAttnError(rc, "decode in drift_report")
        torch.cuda.synchronize()
        t_done = N
        for f in states:
            rows[N]["state"][f"decode_{f}"] = err(widen(states[f], f), S_cp[N])
            rows[N]["output"][f"decode_{f}"] = err(outs[f].float().cpu().numpy(), o_ref[N])
        print(f"[drift] decode reached N={N} ({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)
    return {
        "metric": "stored-state drift vs sequence length (relative max error vs fp64 oracle)",
        "config": {"workload": f"B=1 H={H} N up to {Nmax} d={d}, bf16 q/k/v, prefill block {blk}",
                   "e4m3_scale_per_head": scale.reshape(-1).tolist(), "max_abs_state": smax},
        "data": "synthetic",
        "rows": [rows[N] for N in cps],
        "seconds": time.time() - t0,
    }

if __name__ == "__main__":
    main()
