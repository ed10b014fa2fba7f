// Host-side launch interface of the device kernels (internal to the library;
// the public ABI is include/lin_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lal {

// Storage formats of a state: fp32, or bf16 / OCP FP8 E4M3 codes of
// state / scale.
enum StateFmt { kStF32 = 0, kStBF16 = 1, kStE4M3 = 2 };

// Chunked prefill, bf16 I/O.
struct PrefillArgs {
  const unsigned short *q, *k, *v;  // bf16 bit patterns, [BH][N][d]
  unsigned short *o;
  float *state;                      // [BH][d][d]
  int64_t N;
  int blk;
  int nsplit;   // value-column slices per sequence (d / nsplit columns each)
  int xcd_map;  // set by the launcher
  // optional state snapshots: snap[bh][s] = S after (s + 1) * snap_every
  // full blocks, for s < (N / blk) / snap_every (null: none)
  float *snap;
  int snap_every;
  // narrow-format state (prefill_bf16_scaled_launch; state is then unused):
  // [BH][d][d] codes of state / scale, per-sequence scales (null = 1), and
  // whether the carry is rounded to the format after every block
  void *lp_state;
  const float *lp_scale;
  int lp_round;
  // gradient passes (prefill_bf16_grad_launch; state is then unused): the
  // initial state from g_in (transposed if g_in_t; null = zero), the final
  // state to g_out (null = not stored)
  const float *g_in;
  float *g_out;
  int g_in_t;
  // second pass of a paired gradient launch (prefill_bf16_grad_pair_launch):
  // its q, k, v, o and states, as above
  const unsigned short *q2, *k2, *v2;
  unsigned short *o2;
  const float *g_in2;
  float *g_out2;
  int g_in_t2;
  // one part of a sequence cut along the tokens (prefill_bf16_part_launch):
  // the launch's BH sequences are part_BH sequences of part_P parts each
  // (sequence index = seq * part_P + p); part p starts from part_s0[seq] plus
  // part_sums[c * part_BH + seq] for c < p * part_S, added in that order, and
  // the last part writes its final state to state[seq] (the others to nowhere)
  const float *part_s0;
  const float *part_sums;
  int64_t part_BH;
  int part_P, part_S;
  // one-launch form (prefill_bf16_part_lb_launch, d = 128, part_P <= kPartMaxOneLaunch):
  // part_sums_w (= part_sums) holds 2 (part_P - 1) part_BH d^2 floats: the
  // K^T V of parts 0 .. P-2, then the start states of parts 1 .. P-1, each
  // [part][seq][d^2] in the workgroups' fragment order.  part_flags holds
  // three arrays of part_BH * part_P * kPartMaxSplit words (published,
  // slab, done; [seq][part][slice]), set to part_epoch in turn; the last part
  // clears the words of its slice once every other part is done, so a call
  // leaves the words it used zero.
  float *part_sums_w;
  unsigned long long *part_flags;
  unsigned long long part_epoch;
  unsigned long long part_wait_ticks;  // bound of each wait, in 100 MHz clock ticks
};
constexpr int kPartMaxSplit = 4;
constexpr int kPartMaxOneLaunch = 32;
// Longest wait of a part for a flag of another part (PrefillArgs
// part_wait_ticks), by default: about one second of the 100 MHz constant
// clock (s_memrealtime).  Every awaited part reaches its flag without waiting
// on the waiter, so a wait this long means it could not run; the waiting part
// then poisons what it produces with NaN instead of spinning on.
constexpr unsigned long long kPartWaitTicks = 100000000ull;
// Two reversed gradient passes of the same BH sequences in one launch: pass
// 1 from the q, k, v, o, g_* pointers, pass 2 from the *2 pointers.  The
// two passes must read the same key and value tensors (k2, v2 = v, k); the
// two workgroups of a sequence then run on one XCD and share their tiles
// through its L2.  d = 128 or 64, value columns not split.
hipError_t prefill_bf16_grad_pair_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream);
// The dV and dK passes fused in one reversed sweep per sequence: q tiles
// from k, dout tiles from v (staged once), dV role queries from q with
// outputs to o, dK role queries from q2 with outputs to o2; G from g_in (not
// transposed), dS_0 to g_out.  Value columns not split.
hipError_t prefill_bf16_grad_fused_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream);
int prefill_bf16_max_block(int d);
int prefill_bf16_max_split(int d);
hipError_t prefill_bf16_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream);
// the parts of sequences cut along the tokens (PrefillArgs part_*): BH = part_BH * part_P
hipError_t prefill_bf16_part_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream);
hipError_t prefill_bf16_part_lb_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream);
// state_fmt: kStBF16 or kStE4M3
hipError_t prefill_bf16_scaled_launch(PrefillArgs a, int64_t BH, int d, int state_fmt, hipStream_t stream);
// reverse: walk the sequence from its end (suffix sums)
hipError_t prefill_bf16_grad_launch(PrefillArgs a, int64_t BH, int d, bool reverse, hipStream_t stream);

// Chunked prefill, fp32 I/O.
struct PrefillF32Args {
  const float *q, *k, *v;
  float *o;
  float *state;
  int64_t N;
  int blk;
  float *snap;  // as in PrefillArgs
  int snap_every;
  // gradient passes (grad != 0; state and snap unused): the initial state
  // from g_in (transposed if g_in_t; null = zero), the final state to g_out
  // (null = not stored); rev != 0 takes the tokens in reversed order
  int grad, rev;
  const float *g_in;
  int g_in_t;
  float *g_out;
};
int prefill_f32_max_block(int d);
hipError_t prefill_f32_launch(PrefillF32Args a, int64_t BH, int d, hipStream_t stream);

// One decode token per sequence.
struct DecodeArgs {
  const void *q, *k, *v;
  void *o;
  void *state;         // [BH][d][d] in the storage format
  int64_t BH;
  const float *scale;  // [BH] per-sequence state scale (narrow formats; null = 1)
};
// state_fmt: a StateFmt value (common.hpp)
hipError_t decode_launch(DecodeArgs a, int d, bool io_bf16, int state_fmt, hipStream_t stream);

// Token-by-token prefill with the state on chip.
struct RecurrentArgs {
  const void *q, *k, *v;
  void *o;
  float *state;
  int64_t BH;
  int64_t N;
};
// cus: compute units of the device (the slice width is chosen to fill them)
hipError_t recurrent_launch(RecurrentArgs a, int d, bool io_bf16, int cus, hipStream_t stream);

// Several decode tokens per sequence: verify (outputs, state read only) and
// commit (state += sum over the accepted drafts of k v^T).
struct DecodeMultiArgs {
  const void *q, *k, *v;  // [BH][T][d] of the I/O type
  void *o;
  void *state;            // [BH][d][d]
  const int32_t *accept;  // [B] accepted drafts per batch entry (commit; null = all T)
  int64_t BH;
  int64_t H;
  int T;
  const float *scale;     // [BH] per-sequence state scale (narrow formats; null = 1)
};
int decode_multi_max_tokens();
// state_fmt: a StateFmt value
hipError_t decode_multi_launch(DecodeMultiArgs a, int d, bool commit, bool io_bf16, int state_fmt,
                               hipStream_t stream);

// State accumulation over a token segment: state += K^T V (no q, no outputs).
struct StateDeltaArgs {
  const unsigned short *k, *v;  // bf16 bit patterns, [BH][N][d]
  float *state;                 // [BH][d][d]
  int64_t N;
  int xcd_map;  // set by the launcher
};
hipError_t state_delta_launch(StateDeltaArgs a, int64_t BH, int d, hipStream_t stream);
struct StateDeltaF32Args {
  const float *k, *v;
  float *state;
  int64_t N;
};
hipError_t state_delta_f32_launch(StateDeltaF32Args a, int64_t BH, int d, hipStream_t stream);
// Token-split state accumulation (bf16): chunk c of each sequence covers
// tokens [c chunk_len, min((c+1) chunk_len, N)); chunk 0 adds into state,
// chunks c >= 1 write their sums to partial[(c-1) BH + bh] ([d][d] fp32
// each), which a second launch adds into state in chunk order.
struct StateSplitArgs {
  const unsigned short *k, *v;  // bf16 bit patterns, [BH][N][d]
  float *state;                 // [BH][d][d]
  float *partial;               // [(chunks-1) BH][d][d]
  int64_t N, BH, chunks, chunk_len;
  // non-zero: every chunk c starts from zero and writes partial[c BH + bh]
  // (partial then holds chunks BH states; state is not touched except that
  // the chunk-0 workgroup of each sequence copies state[bh] to s0_copy[bh]
  // when s0_copy is not null)
  int all_partial;
  float *s0_copy;
};
hipError_t state_split_launch(StateSplitArgs a, int d, hipStream_t stream);
// chunks and chunk length (a multiple of 64) for BH sequences of N >= 1 tokens
// on a device of `cus` compute units
void state_split_plan(int64_t BH, int64_t N, int cus, int64_t *chunks, int64_t *chunk_len);

}  // namespace lal
