#!/usr/bin/env python3
"""Benchmark of the causal linear-attention hot path on one MI355X.

One step = one pass over every stage of the path, each on its own batch of
synthetic inputs already resident in HBM:

  * chunked prefill (the headline): B=4, H=64, N=32768, d=128, block 128,
    bf16 q/k/v/o, fp32 state;
  * decode, fp32 state: 256 x 64 sequences, d=128, one token;
  * decode, bf16 state: the same, state stored in bf16;
  * token-by-token prefill and chunked prefill at B=1, H=8, N=4096, d=128,
    block 64 (the crossover comparison), run after a 512 MiB cache flush.

The state buffers are in/out; each step continues from the state the
previous one left (a continuation of longer sequences), which changes no
work.  Every kernel is timed with HIP events on the stream it runs on;
`value` is the chunked prefill's throughput in tokens/s (B*N tokens, all
heads) over the timed steps.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
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

PREFILL_KERNEL_SOURCES = ["linear_attention_lightning_amd/csrc/prefill_bf16.hip",
                          "linear_attention_lightning_amd/csrc/common.hpp"]
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


def cpu_baseline(heads: int = 64, min_seconds: float = 10.0, max_passes: int = 60):
    """The fp64 oracle, timed on this host on a bounded sample of the prefill
    workload: `heads` whole sequences (N = 32768, d = 128; by default the 64
    heads of one batch entry) with the workload's distributions, recomputed
    pass after pass until at least `min_seconds` have elapsed.  Reported in
    the metric's unit: tokens/s, one token being a position of all 64 heads
    (head-tokens/s divided by 64)."""
    from linear_attention_lightning_amd import synth
    from oracle import oracle
    N, d, H = PREFILL["N"], PREFILL["d"], PREFILL["H"]
    q, k, v = synth.prefill_inputs(3, 1, heads, N, d)
    threads = oracle.default_threads()
    oracle.recurrence(q[:, :1, :256], k[:, :1, :256], v[:, :1, :256])  # load + warm the library
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.recurrence(q, k, v, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    head_tokens = heads * N * passes
    return {
        "value": head_tokens / dt / H,
        "unit": "tokens/s",
        "cores": min(threads, heads),
        "kind": "oracle",
        "sample": f"{heads} of the 256 sequences (N=32768, d=128, fp64 token-by-token recurrence), "
                  f"{passes} passes in {dt:.2f} s; {head_tokens * 4 * d * d / dt / 1e9:.1f} GFLOP/s fp64",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--only", choices=["prefill", "decode", "recurrent", "shard", "copy"],
                    help="run one kernel only (for counter collection); prints timings, no JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path shards heads and sequences with no communication, "
              "and this build runs on a single MI355X; use --gpus 1.", file=sys.stderr)
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

    if args.only == "copy":
        # plain copy of a known size, used to calibrate the HBM byte counters
        n = 1 << 30
        x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        for _ in range(args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        print(f"copied {n} bytes x {args.steps}")
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
    if need["decode"]:
        dS32 = synth.decode_initial_state_device(D["B"], D["H"], D["d"])
        dS16 = dS32.to(torch.bfloat16)
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
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    if need["shard"]:
        hq, hk, hv = synth.prefill_inputs_device(4, SH["B"], SH["H"], SH["N"], SH["d"])
        ho = torch.empty_like(hq)
        # a non-zero initial state: the prefix sum of the earlier segments
        hS0 = torch.zeros((SH["B"], SH["H"], SH["d"], SH["d"]), dtype=torch.float32, device=dev)
        la.state_accumulate(hk, hv, hS0)
        hdS = torch.zeros_like(hS0)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    names = [n for n, on in (("prefill", need["prefill"]), ("prefill_snapshots", need["prefill"]),
                             ("decode_fp32", need["decode"]),
                             ("decode_bf16", need["decode"]), ("verify", need["decode"]),
                             ("commit", need["decode"]), ("small_chunked", need["small"]),
                             ("small_recurrent", need["small"]), ("shard_state_accumulate", need["shard"]),
                             ("shard_prefill", need["shard"])) if on]

    def step(evs):
        def timed(name, fn):
            if evs is not None:
                evs[name][0].record(stream)
            fn()
            if evs is not None:
                evs[name][1].record(stream)
        if need["prefill"]:
            timed("prefill", lambda: la.prefill(pq, pk, pv, po, pS, P["block"]))
            timed("prefill_snapshots", lambda: la.prefill_snapshots(pq, pk, pv, po, pS2, psnap, P["block"],
                                                                    SNAP_EVERY))
        if need["decode"]:
            timed("decode_fp32", lambda: la.decode(dq, dk, dv, do, dS32))
            timed("decode_bf16", lambda: la.decode(dq, dk, dv, do, dS16))
            timed("verify", lambda: la.decode_verify(tq, tk, tv, to, dS32))
            timed("commit", lambda: la.decode_commit(tk, tv, dS32, tacc))
        if need["small"]:
            flush.fill_(0)
            timed("small_chunked", lambda: la.prefill(sq, sk, sv, so, sS, S["block"]))
            flush.fill_(1)
            timed("small_recurrent", lambda: la.prefill_recurrent(sq, sk, sv, so2, sS2))
        if need["shard"]:
            timed("shard_state_accumulate", lambda: la.state_accumulate(hk, hv, hdS))
            timed("shard_prefill", lambda: la.prefill(hq, hk, hv, ho, hS0, SH["block"]))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    evs_all = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        evs = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
        step(evs)
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

    p_bytes = prefill_bytes(**P)
    p_flops = prefill_flops(**P)
    p_dense = prefill_dense_flops(**P)
    p_s = avg["prefill"] / 1e3
    tokens = P["B"] * P["N"]
    gbs = p_bytes / p_s / 1e9
    traffic = measured_traffic()
    d32_bytes = decode_bytes(D["B"], D["H"], D["d"], 4)
    d16_bytes = decode_bytes(D["B"], D["H"], D["d"], 2)
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
            "decode_workload": "256 x 64 sequences, d=128, one token per step, fp32 state and bf16 state",
            "crossover_workload": "B=1 H=8 N=4096 d=128 block=64: chunked vs token-by-token",
        },
        "prefill": {
            "ms": avg["prefill"], "ms_min": best["prefill"],
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
        "decode": {
            "fp32_state_ms": avg["decode_fp32"], "fp32_state_GBps": d32_bytes / (avg["decode_fp32"] / 1e3) / 1e9,
            "fp32_state_pct_hbm_peak": 100 * d32_bytes / (avg["decode_fp32"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "bf16_state_ms": avg["decode_bf16"], "bf16_state_GBps": d16_bytes / (avg["decode_bf16"] / 1e3) / 1e9,
            "bf16_state_pct_hbm_peak": 100 * d16_bytes / (avg["decode_bf16"] / 1e3) / 1e9 / PEAK_HBM_GBS,
            "tokens_per_s_fp32_state": D["B"] / (avg["decode_fp32"] / 1e3),
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
            "chunked_tokens_per_s": small_tokens / (avg["small_chunked"] / 1e3),
            "recurrent_tokens_per_s": small_tokens / (avg["small_recurrent"] / 1e3),
            "cache": "each run follows a 512 MiB write that evicts the 256 MB last-level cache",
        },
        "sequence_shard": {
            "workload": "one of 8 segments of the 1M-token sequence: B=1 H=64 N=131072 d=128, bf16",
            "state_accumulate_ms": avg["shard_state_accumulate"],
            "state_accumulate_GBps": state_accumulate_bytes(**SH) / (avg["shard_state_accumulate"] / 1e3) / 1e9,
            "prefill_nonzero_S0_ms": avg["shard_prefill"],
            "prefill_nonzero_S0_GBps": prefill_bytes(**SH) / (avg["shard_prefill"] / 1e3) / 1e9,
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
        },
        "timing": {"wall_ms_timed_region": wall_ms, "setup_s": setup_s,
                   "method": "HIP events on the launch stream around each kernel"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
