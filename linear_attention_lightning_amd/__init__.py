"""Causal linear attention ("Lightning" tiled form) for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``include/lin_attn.h``; this package is the thin Python binding over it
(torch tensors supply device memory and streams) plus the seeded synthetic
input generator used by the tests and the benchmark (``synth``).
"""
from ._binding import (  # noqa: F401
    BWD_AUTO,
    BWD_FUSED,
    BWD_PAIRED,
    BWD_SEPARATE,
    BF16,
    EHIP,
    ESCRATCH,
    EINVAL,
    EUNSUPPORTED,
    F32,
    FP8_E4M3,
    LIB_PATH,
    OK,
    LinAttnError,
    backward,
    decode,
    decode_commit,
    decode_verify,
    library,
    prefill,
    prefill_recurrent,
    prefill_scaled,
    prefill_seqsplit,
    prefill_seqsplit_noalloc,
    prefill_seqsplit_workspace,
    prefill_snapshots,
    scratch_bytes,
    snapshot_count,
    state_accumulate,
    state_accumulate_split,
    state_accumulate_split_workspace,
    strerror,
)

__all__ = ["BWD_AUTO", "BWD_SEPARATE", "BWD_PAIRED", "BWD_FUSED", "prefill", "prefill_scaled", "prefill_seqsplit", "prefill_seqsplit_workspace",
           "prefill_seqsplit_noalloc", "scratch_bytes", "backward", "decode", "decode_verify", "decode_commit", "prefill_recurrent",
           "prefill_snapshots", "snapshot_count", "state_accumulate", "state_accumulate_split",
           "state_accumulate_split_workspace", "strerror", "library", "LinAttnError",
           "F32", "BF16", "FP8_E4M3", "OK", "EINVAL", "EUNSUPPORTED", "EHIP", "ESCRATCH", "LIB_PATH"]
