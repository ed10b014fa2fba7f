/*
 * lin_attn.h -- C ABI of the MI355X (gfx950) causal linear-attention library.
 *
 * The operation.  Causal linear attention with the identity feature map, as
 * defined by its recurrent form in "MiniMax-M1で理解する：大規模言語モデルの
 * コンテキスト長限界を突破する革新的アーキテクチャ" (zenn.dev/liushuzhi),
 * section "線形アテンションの数学的基礎", recurrence equations:
 *
 *     S_t = S_{t-1} + k_t v_t^T            (S in R^{d x d}, fp32)
 *     o_t = q_t^T S_t                      (the token's own k_t v_t^T included)
 *
 * computed in "Lightning" tiles ("Почему M2 в итоге стала моделью с полным
 * вниманием?" (ai.flicky.cc), section 1, glossary entry "Lightning
 * Attention": a masked matrix product inside each block and a K^T V state
 * carried between blocks):
 *
 *     O_b = (Q_b K_b^T ⊙ M) V_b + Q_b S_{b-1},   S_b = S_{b-1} + K_b^T V_b,
 *
 * with M[r][c] = 1 iff c <= r.  The block size changes rounding and speed,
 * never the mathematical result.  No feature map other than the identity, no
 * decay, no normaliser and no 1/sqrt(d) scale is applied.
 *
 * Conventions shared by every entry point.
 *  - Pointers q, k, v, o and state are DEVICE pointers (hipMalloc or
 *    torch-allocated memory on the current HIP device).  The caller owns
 *    every buffer; the library allocates nothing and keeps no per-call state.
 *  - Layouts are dense and row-major: q, k, v, o are [B][H][N][d] (decode:
 *    [B][H][d]); the state is [B][H][d][d] with row i = key feature and
 *    column j = value feature.  Each (b, h) pair is an independent sequence.
 *  - Every base pointer must be 16-byte aligned.  o must not alias q, k or v;
 *    state must not alias any other argument.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous: they enqueue kernels on `stream` and return; o and state
 *    hold the results once that stream has been synchronised.
 *  - All argument checks happen on the host before any HIP call, so a bad
 *    argument returns an error code without touching the device.  Nothing is
 *    thrown across the ABI.  A call with zero work (B*H*N == 0) returns
 *    LIN_ATTN_OK and leaves every buffer untouched.
 *  - The library is reentrant; concurrent calls on different streams are
 *    independent as long as their buffers do not overlap.  The only state it
 *    keeps between calls is a per-device cache of values that never change
 *    while the process runs: the device's compute-unit count (queried once,
 *    used to size grids and split plans) and, for
 *    lin_attn_prefill_seqsplit_noalloc alone, the device address of its fixed
 *    scratch buffer.  Both are written with atomic stores, so concurrent first
 *    calls only repeat the query.
 */
#ifndef LIN_ATTN_H
#define LIN_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v, o and of a stored state. */
typedef enum {
  LIN_ATTN_F32 = 0,      /* IEEE binary32 */
  LIN_ATTN_BF16 = 1,     /* bfloat16; conversions round to nearest, ties to even */
  LIN_ATTN_FP8_E4M3 = 2  /* OCP FP8 E4M3 ("e4m3fn": bias 7, 3 fraction bits, no
                            infinity, largest finite 448); state storage only.
                            Conversions round to nearest, ties to even; finite
                            values beyond +-448 are clamped to +-448; a
                            non-finite value gets an unspecified code */
} lin_attn_dtype_t;

/* Return codes. */
enum {
  LIN_ATTN_OK = 0,
  LIN_ATTN_EINVAL = -1,       /* null pointer with work to do, negative size, misaligned pointer */
  LIN_ATTN_EUNSUPPORTED = -2, /* valid request outside what the kernels implement (d, block, dtype) */
  LIN_ATTN_EHIP = -3,         /* the HIP runtime reported an error (launch or device query) */
  LIN_ATTN_ESCRATCH = -4      /* lin_attn_prefill_seqsplit_noalloc: the plan needs more scratch
                                 memory than the fixed buffer holds (lin_attn_scratch_bytes()) */
};

/*
 * Chunked ("Lightning") prefill over whole sequences.
 *
 * q, k, v : [B][H][N][d] of io_dtype (read only)
 * o       : [B][H][N][d] of io_dtype (written)
 * state   : [B][H][d][d] fp32, IN: S_0 of every sequence, OUT: S_N (in place)
 * block   : tokens per tile.  N need not be a multiple of block; the last
 *           tile of each sequence is partial.
 *
 * Supported: d in {64, 128}.
 *   io_dtype BF16: block a multiple of 16 with 16 <= block <= 128.  All four
 *                  products run on bf16 MFMA with fp32 accumulation; the
 *                  intra-block matrix and the state operand are rounded to
 *                  bf16, the state itself is accumulated in fp32 for the
 *                  whole sequence.
 *   io_dtype F32:  block a multiple of 16 with 16 <= block <= 64 (d = 128)
 *                  or <= 128 (d = 64).  All arithmetic in fp32.
 * Errors: LIN_ATTN_EINVAL, LIN_ATTN_EUNSUPPORTED as above; LIN_ATTN_EHIP if
 * the launch fails.
 */
int lin_attn_prefill(const void *q, const void *k, const void *v, void *o, float *state,
                     int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                     lin_attn_dtype_t io_dtype, void *stream);

/*
 * lin_attn_prefill with an explicit work split.  `split` is the number of
 * value-column slices each sequence is divided into (one workgroup per
 * slice; each slice recomputes the block's Q K^T product).  0 lets the
 * library choose (it splits only while B*H is below the compute-unit count);
 * otherwise bf16 I/O accepts 1, 2 or 4 (d = 128) and 1 or 2 (d = 64), and fp32
 * I/O accepts 1.  Results agree with lin_attn_prefill for every split up to
 * rounding, and are bit-identical across repeated calls with the same split.
 */
int lin_attn_prefill_ex(const void *q, const void *k, const void *v, void *o, float *state,
                        int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                        lin_attn_dtype_t io_dtype, int64_t split, void *stream);

/*
 * lin_attn_prefill that also keeps state snapshots for a prefix cache
 * (resuming a sequence from a stored state is the continuation property of
 * the recurrence; keeping such states is the prefix-caching concern of
 * "ノーフリーランチ" (winzheng.jp), section "推論システム統合の課題").
 *
 * snapshots : [B][H][nsnap][d][d] fp32, written; nsnap = (N / block) / every
 *             (integer divisions).  Snapshot s is S_t, the state after the
 *             first t = (s + 1) * every * block tokens (the initial state
 *             included), i.e. the state a later prefill of the tokens from t
 *             on starts from.  May be NULL when nsnap is 0.
 * every     : blocks between snapshots, >= 1 (else LIN_ATTN_EINVAL).
 *
 * All other arguments, results and errors as lin_attn_prefill; o and the
 * final state are bit-identical to lin_attn_prefill's.
 */
int lin_attn_prefill_snapshots(const void *q, const void *k, const void *v, void *o, float *state,
                               float *snapshots, int64_t B, int64_t H, int64_t N, int64_t d,
                               int64_t block, int64_t every, lin_attn_dtype_t io_dtype, void *stream);

/*
 * Chunked prefill with the state stored in a narrow format under a
 * per-sequence scale (the storage of lin_attn_decode_scaled), for a state
 * cache that keeps states in bf16 or FP8 between calls.
 *
 * state       : [B][H][d][d] of state_dtype (LIN_ATTN_BF16 or
 *               LIN_ATTN_FP8_E4M3), IN: the stored S_0, OUT: the stored S_N.
 * state_scale : DEVICE pointer to float[B][H], or NULL (as for
 *               lin_attn_decode_scaled); the same scale reads S_0 and stores
 *               S_N.
 * round_carry : 0: the carry between blocks stays in fp32 and only S_N is
 *               rounded, on its store.
 *               1: the carry is rounded to state_dtype after every block
 *               (the partial last block included), as if the sequence were
 *               prefilled one block per call with the state stored in between;
 *               each block's outputs read the rounded carry of the blocks
 *               before it.
 *               Other values: LIN_ATTN_EINVAL.
 *
 * Everything else as lin_attn_prefill (work split chosen by the library).
 * Supported: io_dtype BF16 only, d in {64, 128}, block as for bf16 in
 * lin_attn_prefill.
 */
int lin_attn_prefill_scaled(const void *q, const void *k, const void *v, void *o, void *state,
                            const float *state_scale, int64_t B, int64_t H, int64_t N, int64_t d,
                            int64_t block, lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype,
                            int64_t round_carry, void *stream);

/*
 * One decode token per sequence: S <- S + k v^T, then o = q^T S (the
 * recurrence above with N = 1), for all B*H sequences at once.
 *
 * q, k, v : [B][H][d] of io_dtype (read only)
 * o       : [B][H][d] of io_dtype (written)
 * state   : [B][H][d][d] of state_dtype, updated in place.  With
 *           state_dtype = LIN_ATTN_BF16 the state is widened to fp32, updated
 *           in fp32, o is read from the fp32 value, and the state is stored
 *           back rounded to bf16 (the low-precision state storage discussed in
 *           "ノーフリーランチ：MiniMax M2が高効率アテンション機構を解体"
 *           (winzheng.jp), section "推論システム統合の課題").
 *
 * Supported: d in {64, 128}; io_dtype in {F32, BF16}; state_dtype in {F32,
 * BF16, FP8_E4M3} (FP8_E4M3 as in lin_attn_decode_scaled with unit scales).
 */
int lin_attn_decode(const void *q, const void *k, const void *v, void *o, void *state,
                    int64_t B, int64_t H, int64_t d,
                    lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream);

/*
 * Decode step with the state stored in a narrow format under a per-sequence
 * scale (FP8 or other low-precision storage of a state that is rewritten
 * every token: "ノーフリーランチ" (winzheng.jp), section "推論システム統合の
 * 課題").
 *
 * state       : [B][H][d][d] of state_dtype (LIN_ATTN_BF16 or
 *               LIN_ATTN_FP8_E4M3), updated in place.  Entry x of sequence
 *               (b, h) is held as the code of x / scale[b][h]; its value is
 *               value(code) * scale[b][h].
 * state_scale : DEVICE pointer to float[B][H], or NULL for 1.0 everywhere.
 *               Scales must be positive and finite (others give unspecified
 *               results, never a fault); with powers of two the scaling is
 *               exact and the result is that of the unscaled computation on
 *               scaled values.
 *
 * Per sequence: the stored state is widened to fp32, S += k v^T in fp32, o is
 * read from the fp32 value, and the state is stored back rounded to
 * state_dtype (conversion rules at lin_attn_dtype_t).  lin_attn_decode with
 * state_dtype BF16 or FP8_E4M3 is this call with state_scale = NULL.
 *
 * Supported: d in {64, 128}; io_dtype in {F32, BF16}; state_dtype in {BF16,
 * FP8_E4M3} (LIN_ATTN_F32: LIN_ATTN_EUNSUPPORTED, use lin_attn_decode).
 */
int lin_attn_decode_scaled(const void *q, const void *k, const void *v, void *o, void *state,
                           const float *state_scale, int64_t B, int64_t H, int64_t d,
                           lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream);

/*
 * Verification of T draft tokens per sequence (speculative decoding):
 * o_t = q_t^T S_t for t = 0 .. T-1 with S_t = S + sum_{s <= t} k_s v_s^T,
 * i.e. the outputs T decode steps would produce, from one read of the state,
 * which is NOT modified.  Once the caller knows how many drafts each
 * sequence accepts, lin_attn_decode_commit advances the state by exactly
 * those ("ノーフリーランチ" (winzheng.jp), section "推論システム統合の課題",
 * names draft verification and rollback as open problems of linear
 * attention; here a rollback is simply a commit of 0 tokens).
 *
 * q, k, v, o : [B][H][T][d] of io_dtype (o written)
 * state      : [B][H][d][d] of state_dtype, read only
 * T          : 0 .. 16 (0 is a no-op; larger values: LIN_ATTN_EUNSUPPORTED)
 *
 * Supported: d in {64, 128}; io_dtype in {F32, BF16}; state_dtype in {F32,
 * BF16, FP8_E4M3} (FP8_E4M3 with unit scales; see lin_attn_decode_verify_scaled).
 */
int lin_attn_decode_verify(const void *q, const void *k, const void *v, void *o, const void *state,
                           int64_t B, int64_t H, int64_t T, int64_t d,
                           lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream);

/*
 * Commit of accepted drafts: S <- S + sum_{t < a_b} k_t v_t^T for every head
 * of batch entry b, with a_b = accept[b] clamped to [0, T].
 *
 * k, v   : [B][H][T][d] of io_dtype (the drafts given to lin_attn_decode_verify)
 * state  : [B][H][d][d] of state_dtype, updated in place
 * accept : DEVICE pointer to int32[B], or NULL to accept all T drafts
 *
 * With an fp32 state the result is bit-identical to a_b calls of
 * lin_attn_decode (same operations in the same order); with a bf16 or
 * FP8_E4M3 state the update is done in fp32 and rounded once, at the store.
 * Errors and limits as lin_attn_decode_verify.
 */
int lin_attn_decode_commit(const void *k, const void *v, void *state, const int32_t *accept,
                           int64_t B, int64_t H, int64_t T, int64_t d,
                           lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream);

/*
 * lin_attn_decode_verify and lin_attn_decode_commit for a state stored in a
 * narrow format under per-sequence scales (the storage of
 * lin_attn_decode_scaled: entry x held as the code of x / scale[b][h]).
 * state_scale is a DEVICE pointer to float[B][H], or NULL for 1.0.  Verify
 * reads the widened state; commit widens, adds the accepted drafts in fp32
 * and rounds once at the store.
 *
 * Supported: as the unscaled calls, with state_dtype in {BF16, FP8_E4M3}
 * (LIN_ATTN_F32: LIN_ATTN_EUNSUPPORTED).
 */
int lin_attn_decode_verify_scaled(const void *q, const void *k, const void *v, void *o, const void *state,
                                  const float *state_scale, int64_t B, int64_t H, int64_t T, int64_t d,
                                  lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream);
int lin_attn_decode_commit_scaled(const void *k, const void *v, void *state, const float *state_scale,
                                  const int32_t *accept, int64_t B, int64_t H, int64_t T, int64_t d,
                                  lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream);

/*
 * Token-by-token prefill: the recurrence above applied one token at a time
 * inside one kernel, with the fp32 state held on chip and plain vector FMAs
 * (4 d^2 flop per token, no matrix cores).  Same arguments, layouts and
 * results as lin_attn_prefill, without the block argument; it is the
 * sequential baseline the tiled form is compared against ("ノーフリーランチ"
 * (winzheng.jp), section "計算とメモリのボトルネックの不整合": the expected
 * break-even of linear attention at a few thousand tokens).
 *
 * Supported: d in {64, 128}; io_dtype in {F32, BF16}.
 */
int lin_attn_prefill_recurrent(const void *q, const void *k, const void *v, void *o,
                               float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                               lin_attn_dtype_t io_dtype, void *stream);

/*
 * State accumulation over a token segment: state <- state + K^T V, i.e. the
 * state update of the recurrence above applied to N tokens, without q and
 * without outputs.  Summed in front of a later segment, the result is that
 * segment's initial state: a sequence cut into segments processed
 * independently is recombined by exclusive prefix sums of their K^T V
 * (the decomposition implied by the associativity equation of [ZENN],
 * section "線形アテンションの数学的基礎").
 *
 * k, v  : [B][H][N][d] of io_dtype (read only)
 * state : [B][H][d][d] fp32, updated in place (start from zero to obtain
 *         K^T V alone)
 *
 * Supported: d in {64, 128}; io_dtype in {F32, BF16}.  bf16 products run on
 * matrix cores with fp32 accumulation; the result is deterministic (fixed
 * summation order, no atomics).
 */
int lin_attn_state_accumulate(const void *k, const void *v, float *state,
                              int64_t B, int64_t H, int64_t N, int64_t d,
                              lin_attn_dtype_t io_dtype, void *stream);

/*
 * The same state accumulation, cut along the tokens: each sequence's N
 * tokens are split into chunks, one workgroup per (sequence, chunk) sums its
 * chunk's K^T V over the whole d x d state, and the chunk sums are added to
 * the state in chunk order (so the result is deterministic, and equal to the
 * call above up to fp32 rounding).  Every K and V byte is then read once, as
 * whole rows, by one workgroup; the call above reads each byte once per
 * 64 x 64 tile row or column of the state that needs it.  The chunk sums
 * other than the first go to a caller-provided workspace.
 *
 * lin_attn_state_accumulate_split_workspace returns the workspace bytes the
 * call needs for these sizes on the current device (the chunk count depends
 * on its compute-unit count; 0 when a single chunk per sequence suffices,
 * and for fp32 I/O, which runs the unsplit kernel), or a negative error code
 * (LIN_ATTN_EINVAL, LIN_ATTN_EUNSUPPORTED) for arguments the call rejects, or
 * LIN_ATTN_EHIP when the device cannot be queried.
 *
 * workspace       : device pointer, 16-byte aligned, at least that many
 *                   bytes, owned by the caller, not aliasing k, v or state;
 *                   may be NULL when 0 bytes are needed.  Its contents on
 *                   entry are ignored and on return unspecified.
 * workspace_bytes : its size; fewer bytes than needed give LIN_ATTN_EINVAL.
 * Other arguments and errors as lin_attn_state_accumulate.  Calls that share
 * a workspace must not run concurrently.
 */
int64_t lin_attn_state_accumulate_split_workspace(int64_t B, int64_t H, int64_t N, int64_t d,
                                                  lin_attn_dtype_t io_dtype);
int lin_attn_state_accumulate_split(const void *k, const void *v, float *state,
                                    int64_t B, int64_t H, int64_t N, int64_t d,
                                    lin_attn_dtype_t io_dtype, void *workspace,
                                    int64_t workspace_bytes, void *stream);

/*
 * Prefill cut along the tokens, for few sequences: the same outputs and
 * final state as lin_attn_prefill (up to fp32 rounding of the carried
 * state), computed as follows.  Each sequence's N tokens are cut into P equal
 * parts so that B*H*P is at most the device's compute-unit count (one
 * chunked-prefill workgroup per compute unit, before any value-column split;
 * parts of at least 256 tokens, P a power of two dividing N).  Each part
 * starts from S_0 plus the K^T V sums of the parts before it, added in part
 * order (the associativity equation of [ZENN], section
 * "線形アテンションの数学的基礎": the state after a concatenation is the sum
 * of the segments' K^T V), and runs as a chunked prefill; the last part of
 * each sequence writes the final state to state.
 *  - d = 128 and P <= 32: one launch.  Each part but the last first sums K^T V over its
 *    own tokens and publishes the sum; the parts of a sequence then form the
 *    start states together (each for 1/P of the state's elements) and
 *    publish them; each part reads its own start and runs.  Parts wait for
 *    one another through flags in the workspace, which hold a per-call
 *    random 64-bit value when set; a wait longer than about one second
 *    (only possible when the parts of a launch cannot all run, e.g. a device
 *    shared with a kernel that never yields) gives NaN outputs instead of
 *    hanging.  The environment variable LIN_ATTN_PART_WAIT_TICKS, read at
 *    each call, sets that bound in ticks of the 100 MHz constant clock (a
 *    test setting: 0 makes waits run out).
 *  - otherwise two launches.  The token-split accumulation sums the K^T V of
 *    the first P-1 parts into the workspace (which also receives a copy of
 *    S_0); the parts then run as B*H*P prefills, each adding the sums of the
 *    parts before it itself.
 * Both read K and V once more for (P-1)/P of the tokens, and in exchange
 * fill the GPU where B*H alone would leave compute units idle.  When P = 1
 * (enough sequences, short or indivisible N, or fp32 I/O) the call is
 * lin_attn_prefill and needs no workspace.
 *
 * lin_attn_prefill_seqsplit_workspace returns the workspace bytes the call
 * needs on the current device (the plan depends on its compute-unit count):
 * 2 (P-1) * B*H * d*d * 4 + 96 * B*H*P for one launch, ((P-1) S + 1) * B*H
 * * d*d * 4 for two launches with S <= 4 accumulation chunks per part, 0
 * when P = 1; or a negative error code for arguments the call rejects
 * (LIN_ATTN_EHIP when the device cannot be queried).  The workspace's
 * contents on entry do not matter, and a call leaves its flag words zero;
 * calls that overlap in time must not share a workspace.
 * workspace, workspace_bytes: as lin_attn_state_accumulate_split.  Other
 * arguments, layouts and errors as lin_attn_prefill.
 */
int64_t lin_attn_prefill_seqsplit_workspace(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                                            lin_attn_dtype_t io_dtype);
int lin_attn_prefill_seqsplit(const void *q, const void *k, const void *v, void *o, float *state,
                              int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                              lin_attn_dtype_t io_dtype, void *workspace, int64_t workspace_bytes,
                              void *stream);

/*
 * lin_attn_prefill_seqsplit for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc.  The same plan, kernels and results as
 * lin_attn_prefill_seqsplit (bitwise), with the workspace taken from a fixed
 * buffer inside the library instead of an argument.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 * The buffer: lin_attn_scratch_bytes() bytes (56 MiB) of device memory per
 * device the library runs on, held from the library's load until the process
 * ends.  Its device address is looked up once per device, on the first call
 * on that device.  Every call on a device uses that device's one buffer, and
 * nothing in it needs to start at zero: each byte the kernels read was written
 * earlier in the same call, except the one-launch plan's flag words, which
 * count as set only when they hold that call's random 64-bit value (and
 * which each call leaves zero).  Calls that overlap in time on one device
 * (different streams, or different host threads) therefore race on the
 * buffer and give wrong results: serialise them, e.g. on one stream.
 *
 * Errors: as lin_attn_prefill_seqsplit, with no workspace arguments, plus
 * LIN_ATTN_ESCRATCH when the plan for these sizes needs more than
 * lin_attn_scratch_bytes() of workspace (lin_attn_prefill_seqsplit_workspace
 * gives the amount); that check runs before any launch.
 */
int64_t lin_attn_scratch_bytes(void);
int lin_attn_prefill_seqsplit_noalloc(const void *q, const void *k, const void *v, void *o, float *state,
                                      int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                                      lin_attn_dtype_t io_dtype, void *stream);

/*
 * Backward pass (training): the gradients of L = sum_t <o_t, dout_t> +
 * <S_N, dstate> through the prefill above, for upstream gradients dout of
 * the outputs and dstate of the final state.  With the gradient reaching S_t,
 * G_t = dstate + sum_{r >= t} q_r dout_r^T (the chain rule through the
 * recurrence of [ZENN], section "線形アテンションの数学的基礎"):
 *
 *     dq_t = S_t dout_t,   dk_t = G_t v_t,   dv_t = G_t^T k_t,   dstate0 = G_0.
 *
 * In block form these are the prefill itself in other roles: dQ is the
 * prefill of (dout, V, K) from S_0^T, and dV and dK are prefills of
 * (K, Q, dout) from dstate and of (V, dout, Q) from dstate^T taken over the
 * reversed token order (suffix sums); the first of those ends in dstate0.
 * dV and dK share their keys and values (q and dout, swapped) and the carried
 * state (G and G^T): when the B*H sequences fill the GPU without splitting
 * value columns, they run fused, one reversed sweep per sequence that stages
 * each q and dout tile once for both (strategy LIN_ATTN_BWD_FUSED below);
 * otherwise as separate passes.  All launches go on `stream`.
 *
 * q, k, v, dout  : [B][H][N][d] of io_dtype (read only)
 * state0         : [B][H][d][d] fp32, the S_0 of the forward call, or NULL
 *                  (zero); read only
 * dstate         : [B][H][d][d] fp32 gradient of the final state, or NULL
 *                  (zero); read only
 * dq, dk, dv     : [B][H][N][d] of io_dtype (written)
 * dstate0        : [B][H][d][d] fp32 gradient of S_0 (written), or NULL
 * block          : as lin_attn_prefill
 *
 * No output may alias an input or another output.
 * Supported: io_dtype BF16 or F32, d in {64, 128}, block as lin_attn_prefill
 * allows for that dtype.  With bf16 I/O the products run on bf16 matrix cores
 * with fp32 accumulation (the carried states in fp32), as in the forward
 * kernel; with fp32 I/O every product and sum is fp32 on the vector ALUs (the
 * fp32 prefill kernel in the same roles, three launches).
 */
int lin_attn_backward(const void *q, const void *k, const void *v, const void *dout,
                      const float *state0, const float *dstate, void *dq, void *dk, void *dv,
                      float *dstate0, int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                      lin_attn_dtype_t io_dtype, void *stream);

/*
 * lin_attn_backward with the way the dV and dK passes run chosen by the
 * caller (the results agree to fp32 rounding of the carried states; the
 * separate, paired and fused forms give bitwise equal gradients):
 *   LIN_ATTN_BWD_AUTO     as lin_attn_backward;
 *   LIN_ATTN_BWD_SEPARATE two launches, value columns split while B*H alone
 *                         leaves compute units idle;
 *   LIN_ATTN_BWD_PAIRED   one launch of 2*B*H workgroups: a sequence's dV and
 *                         dK workgroups share an XCD and read the same q and
 *                         dout tiles, the second reader served by its L2;
 *   LIN_ATTN_BWD_FUSED    one workgroup per sequence computes both.
 * Any other value gives LIN_ATTN_EINVAL.  Other arguments as lin_attn_backward.
 */
enum { LIN_ATTN_BWD_AUTO = 0, LIN_ATTN_BWD_SEPARATE = 1, LIN_ATTN_BWD_PAIRED = 2, LIN_ATTN_BWD_FUSED = 3 };
int lin_attn_backward_ex(const void *q, const void *k, const void *v, const void *dout,
                         const float *state0, const float *dstate, void *dq, void *dk, void *dv,
                         float *dstate0, int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                         lin_attn_dtype_t io_dtype, int64_t strategy, void *stream);

/* Static, human-readable text for a return code (never NULL). */
const char *lin_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* LIN_ATTN_H */
