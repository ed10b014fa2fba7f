"""Host logic of bench.py, checked without a GPU: the algorithmic byte and
flop models against independent counts, the guard on the counter summary
that supplies roofline.traffic, and the one-GPU rule of --gpus."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_byte_and_flop_models():
    P = bench.PREFILL
    # 4 tensors of B*H*N*d bf16 values (q, k, v in, o out) plus the fp32
    # state read and written once per sequence
    elems = P["B"] * P["H"] * P["N"] * P["d"]
    assert bench.prefill_bytes(**P) == 4 * elems * 2 + 2 * P["B"] * P["H"] * P["d"] ** 2 * 4
    assert bench.prefill_bytes(**P) == 8_623_489_024
    # useful flop: per token, the readout q^T S (2 d^2), the update k v^T
    # (2 d^2) and the causal intra-block part, summed exactly over the
    # positions of a block: token r of a block sees r + 1 keys (2 d flop for
    # the score, 2 d for the value), averaged over the block = 2 d (blk + 1)
    d, blk = P["d"], P["block"]
    intra = sum(2 * d * (r + 1) * 2 for r in range(blk)) / blk
    assert intra == 2 * d * (blk + 1)
    per_token = 4 * d * d + intra
    assert bench.prefill_flops(**P) == P["B"] * P["H"] * P["N"] * per_token
    # dense: the full blk x blk masked tile for both products
    assert bench.prefill_dense_flops(**P) == P["B"] * P["H"] * P["N"] * (4 * d * d + 4 * d * blk)


def test_other_byte_models():
    D = bench.DECODE
    heads = D["B"] * D["H"]
    # decode: the state read and written once, q, k, v read and o written
    assert bench.decode_bytes(D["B"], D["H"], D["d"], 4) == heads * (2 * D["d"] ** 2 * 4 + 4 * D["d"] * 2)
    assert bench.decode_bytes(D["B"], D["H"], D["d"], 4) == heads * 132_096
    assert bench.decode_bytes(D["B"], D["H"], D["d"], 1) == heads * 33_792
    S = bench.SHARD
    assert bench.state_accumulate_bytes(**S) == S["B"] * S["H"] * (S["N"] * 2 * S["d"] * 2 + 2 * S["d"] ** 2 * 4)
    P = bench.PREFILL
    # the least a backward moves: q, k, v, dO in and dq, dk, dv out (bf16),
    # and the fp32 gradient of S_0 out
    elems = P["B"] * P["H"] * P["N"] * P["d"]
    assert bench.backward_bytes(**P) == 7 * elems * 2 + P["B"] * P["H"] * P["d"] ** 2 * 4
    # the default's two launches: dQ (3 in, 1 out) + fused dK/dV (4 in, 2 out)
    assert bench.backward_design_bytes(**P) == 10 * elems * 2 + P["B"] * P["H"] * P["d"] ** 2 * 4


def test_traffic_only_for_the_recorded_sources(tmp_path, monkeypatch):
    """roofline.traffic comes from the counter summary only while the kernel
    sources hash to the value recorded in it."""
    good = bench.source_hash(bench.PREFILL_KERNEL_SOURCES)
    summary = tmp_path / "summary.md"
    summary.write_text(f"kernel source hash: `{good}`\ncalibrated HBM bytes per launch: `8.5e+09`\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    assert bench.measured_traffic() == 8.5e9
    summary.write_text("kernel source hash: `0123456789abcdef`\ncalibrated HBM bytes per launch: `8.5e+09`\n")
    assert bench.measured_traffic() is None
    summary.unlink()
    assert bench.measured_traffic() is None


def test_committed_summary_matches_the_sources():
    """The committed counter summary was taken on the kernel sources as they
    stand (else roofline.traffic would be null in the bench line)."""
    assert bench.measured_traffic() is not None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
