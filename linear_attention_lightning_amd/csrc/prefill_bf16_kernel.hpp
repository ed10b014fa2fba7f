// Chunked ("Lightning") causal linear-attention prefill on bf16 matrix cores:
// the kernel template, included by the translation units that instantiate it.
//
// Method: "Почему M2 в итоге стала моделью с полным вниманием?"
// (ai.flicky.cc), section 1, glossary entry "Lightning Attention" -- linear
// attention computed in tiles, with a masked matrix product inside each block
// and a K^T V state carried between blocks -- applied to the recurrence
// S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t of "MiniMax-M1で理解する…"
// (zenn.dev/liushuzhi), section "線形アテンションの数学的基礎".  Per block b of
// `blk` tokens (M[r][c] = 1 iff c <= r):
//
//   O_b = (Q_b K_b^T ⊙ M) V_b + Q_b S_{b-1}          (read S before the update)
//   S_b = S_{b-1} + K_b^T V_b
//
// Work decomposition.  One workgroup (4 waves) owns one (batch, head)
// sequence and a slice of DV value columns [j0, j0 + DV); it walks the blocks
// of its sequence in order.  The fp32 state slice lives in matrix-core
// accumulators for the whole sequence and is copied to LDS as bf16 once per
// block, as the operand of Q_b S.  Slices of one sequence recompute Q_b K_b^T
// each; they exist to fill the GPU when B*H is small.
//
// Data movement (gfx950):
//  * K and V tiles go HBM -> LDS with buffer_load ... lds (no registers),
//    double-buffered: block b+1 streams in while block b is computed.  The
//    buffer descriptor covers exactly the valid rows, so rows past the end of
//    the sequence arrive as zeros -- ragged tails need no other masking.
//  * Q rows are loaded by each wave into registers one block ahead, as whole
//    128-byte lines (one L1 request per line), and rearranged into the
//    matrix-core operand layout by a masked DPP row rotation; the head
//    dimension is contracted in the chunk order that this layout gives, for
//    all operands alike.
//  * K, V and Q are read once, with the non-temporal cache policy.
//  * LDS tiles are unpadded with an XOR swizzle of their 16-byte chunks,
//    chosen so that 16-byte fragment reads (one row per lane) and the
//    transposing 8-byte reads both run without bank conflicts.
//
// Products (all v_mfma_f32_16x16x32_bf16).  Outputs are computed transposed,
// O^T = S^T Q^T + V^T P^T, so a lane holds four consecutive value features of
// one token; lane swaps across value tiles (permlane32/16 swaps, a DPP row
// rotation) turn them into 16-byte stores that write whole 128-byte lines.
// P^T = K Q^T lands directly in the B-operand layout of V^T P^T.  K^T and V
// are read token-major with ds_read_b64_tr_b16.
//
// Balance.  Phase A (outputs) pairs row tiles t and NT-1-t so that every
// wave has the same causal work, and splits value columns across the waves
// of a pair; phase B (state update) spreads the state over the waves by row
// tiles.  The number of 16-row tiles per block, NT, is a template parameter
// so that every loop bound is a compile-time constant.
//
// Reversed traversal (SM = kPsGradRev) walks the blocks from the end of the
// sequence and reads each block's rows in reverse: logical row r of a block
// is the token len-1-r of its span in memory.  The causal mask then keeps
// the tokens at or after each token, so the same kernel computes suffix
// sums -- the reverse-carried state of the gradients.  Every buffer offset
// of a row stays in the per-lane offset register; rows past the block's end
// get negative offsets, which lie outside the buffer descriptor, so they
// read zeros and their stores are dropped, as in forward order.  The dV and
// dK passes of the gradients share their keys and values (q and dout,
// swapped) and their carried states (G and G^T): kPsGradRevPair runs both
// passes in one launch with a sequence's two workgroups on one XCD, and
// kPsGradFused runs both in one workgroup that stages each tile once.
//
// State storage (template parameter SM).  The state that enters and leaves
// the kernel is fp32, optionally with snapshots of it every few blocks (a
// prefix cache), or codes of state / scale in bf16 or OCP FP8 E4M3 (a state
// cache in a narrow format, "ノーフリーランチ" (winzheng.jp), section
// "推論システム統合の課題").  With a narrow format the carry may also be
// rounded to it after every block, which is what prefilling one block per
// call with the state stored in between would compute.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kWaves = 4;  // one per SIMD, each with the whole register file
constexpr int kThreads = kWaves * 64;
constexpr int kBlkMax = 128;
// Cache policy of the output stores: non-temporal (each output byte is
// written once and not read back by the kernel).  Measured 5 % faster than
// the default policy on the largest prefill, with the stores spread over the
// state update: the write stream then leaves L2 without displacing lines.
constexpr int kStNT = 2;

enum PrefillStateMode {
  kPsF32 = 0,      // fp32 state in and out
  kPsF32Snap = 1,  // fp32 state plus snapshots
  kPsBF16 = 2,     // bf16 codes of state / scale
  kPsE4M3 = 3,     // OCP FP8 E4M3 codes of state / scale
  kPsGrad = 4,     // fp32 state from g_in (optionally transposed, null = 0) to g_out (null: none)
  kPsGradRev = 5,  // as kPsGrad, with the token order reversed (suffix sums instead of prefix sums)
  // as kPsGradRev, two passes in one launch: the workgroups of a sequence's
  // two passes (value slice 0 and 1 of the nsplit = 2 mapping, the second
  // with the *2 pointers) share an XCD and stream the same K and V tiles,
  // which they load with the default cache policy so that L2 can serve the
  // second reader
  kPsGradRevPair = 6,
  // the dV and dK passes fused (reversed order, value columns not split): the
  // K and V tiles staged in LDS are those of q and dout, read once for both;
  // the dV role takes the k rows as queries and the carried state G as is,
  // the dK role the v rows and G transposed (q2 = v rows, o2 = dk)
  kPsGradFused = 7,
  // one part of a sequence cut along the tokens: fp32 initial state formed
  // from the sequence's S_0 and the K^T V sums of the parts before it; only
  // the last part stores its final state (PrefillArgs part_*)
  kPsPart = 8,
  // as kPsPart, with the parts' K^T V sums formed in the same launch: each
  // part but the last first sums K^T V over its own tokens and publishes it
  // behind a flag; each part then adds the published sums of the parts
  // before it, in part order (PrefillArgs part_flags, part_epoch)
  kPsPartLB = 9
};


// Round x / scale to the storage format of SM and return the stored value
// times scale (exact for power-of-two scales).
template <int SM>
__device__ __forceinline__ f32x4 round_to_store(f32x4 x, float sc, float inv) {
  f32x4 r;
  if constexpr (SM == kPsBF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (float)(bf16)(x[e] * inv) * sc;
  } else {
    const f32x4 y = {x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
    r = e4m3x4_to_f32(f32_to_e4m3x4(y));
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] *= sc;
  }
  return r;
}

// Physical 16-byte chunk of logical chunk c in row r of a tile whose rows
// hold CPR chunks (an involution).  gfx950's LDS serves a 16-byte read of a
// half wave (32 lanes) in two cycles when no 16-byte bank slot (address / 16
// mod 16) is hit more than twice, and an 8-byte read of a half wave in one
// cycle when all 64 banks differ (measured with a bank-conflict probe).  The
// fragment reads of 256-byte rows (lane groups of 16 lanes on rows r..r+15,
// one logical chunk) then need 16 distinct slots over any 16 consecutive
// rows, and the transposing reads (8 consecutive rows, two adjacent logical
// chunks each) 8 distinct slot pairs: XOR with 2 (r mod 8) + (r / 8 mod 2)
// gives both.  Rows of 128 and 64 bytes put 2 and 4 rows in one 256-byte
// slot window, and their XORs give both properties too.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR == 16)
    return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
  else if constexpr (CPR == 8)
    return c ^ ((r >> 1) & 7);
  else
    return c ^ ((r >> 2) & 3);
}

// Element offset of (row r, column col), col a multiple of 4, in such a tile.
template <int CPR>
__device__ __forceinline__ int sw_off(int r, int col) {
  return r * (CPR * 8) + (swz<CPR>(r, col >> 3) << 3) + (col & 7);
}

// Workgroup barrier that waits only for this wave's outstanding LDS accesses
// (not for vector-memory loads).  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 8-byte LDS store the compiler does not track.  Its ordering against
// in-flight direct loads is guaranteed by construction (they target other
// buffers), and its completion by the lgkmcnt(0) of the next lds_barrier().
__device__ __forceinline__ void lds_store_b64(const void *lds_ptr, uint2 v) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) const char *)lds_ptr;
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Raw buffer descriptor as four scalar words: `bytes` bytes from `base`,
// stride 0, 32-bit data format; accesses at or past `bytes` read zero.
__device__ __forceinline__ u32x4 raw_desc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// Direct HBM -> LDS load of 16 bytes per lane: lane l's bytes at `voff` in
// the buffer land at LDS byte address lds_base + 16 l.  The load is marked
// non-temporal (the tile is read once): measured 3 % faster at the largest
// workloads than the default policy.  Issued from inline
// assembly so that the compiler does not track it: its own vector-memory
// waits would otherwise drain these loads before every LDS read, even of
// other buffers.  Its completion is awaited explicitly with wait_vmcnt()
// followed by a barrier.  M0 holds the LDS base; one wait state separates its
// write from the load that reads it.
// M0 is a reserved register; clobbering it is sound here because nothing else
// in these kernels keeps a value in M0 (no other LDS-DMA, message or
// relative-addressing instruction is generated).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128(u32x4 desc, int voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voff), "s"(desc), "s"(lds_base) : "memory", "m0");
}
// the same with the default cache policy (tiles that a second workgroup reads)
__device__ __forceinline__ void dma_b128_shared(u32x4 desc, int voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(desc), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of p as a scalar.  The zero added comes from an
// instruction with side effects, so the sum is formed where it is used rather
// than kept in a scalar register for the whole kernel.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  unsigned zero;
  asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
  return zero + __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) const char *)p);
}

// Wait until at most n vector-memory operations of this wave are in flight
// (they complete in issue order).
__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt takes an immediate (6 bits): dispatch over every count
  switch (n) {
#define LAL_WAIT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    LAL_WAIT_CASE(0) LAL_WAIT_CASE(1) LAL_WAIT_CASE(2) LAL_WAIT_CASE(3) LAL_WAIT_CASE(4) LAL_WAIT_CASE(5) LAL_WAIT_CASE(6) LAL_WAIT_CASE(7)
    LAL_WAIT_CASE(8) LAL_WAIT_CASE(9) LAL_WAIT_CASE(10) LAL_WAIT_CASE(11) LAL_WAIT_CASE(12) LAL_WAIT_CASE(13) LAL_WAIT_CASE(14) LAL_WAIT_CASE(15)
    LAL_WAIT_CASE(16) LAL_WAIT_CASE(17) LAL_WAIT_CASE(18) LAL_WAIT_CASE(19) LAL_WAIT_CASE(20) LAL_WAIT_CASE(21) LAL_WAIT_CASE(22) LAL_WAIT_CASE(23)
    LAL_WAIT_CASE(24) LAL_WAIT_CASE(25) LAL_WAIT_CASE(26) LAL_WAIT_CASE(27) LAL_WAIT_CASE(28) LAL_WAIT_CASE(29) LAL_WAIT_CASE(30) LAL_WAIT_CASE(31)
    LAL_WAIT_CASE(32) LAL_WAIT_CASE(33) LAL_WAIT_CASE(34) LAL_WAIT_CASE(35) LAL_WAIT_CASE(36) LAL_WAIT_CASE(37) LAL_WAIT_CASE(38) LAL_WAIT_CASE(39)
    LAL_WAIT_CASE(40) LAL_WAIT_CASE(41) LAL_WAIT_CASE(42) LAL_WAIT_CASE(43) LAL_WAIT_CASE(44) LAL_WAIT_CASE(45) LAL_WAIT_CASE(46) LAL_WAIT_CASE(47)
    LAL_WAIT_CASE(48) LAL_WAIT_CASE(49) LAL_WAIT_CASE(50) LAL_WAIT_CASE(51) LAL_WAIT_CASE(52) LAL_WAIT_CASE(53) LAL_WAIT_CASE(54) LAL_WAIT_CASE(55)
    LAL_WAIT_CASE(56) LAL_WAIT_CASE(57) LAL_WAIT_CASE(58) LAL_WAIT_CASE(59) LAL_WAIT_CASE(60) LAL_WAIT_CASE(61) LAL_WAIT_CASE(62) LAL_WAIT_CASE(63)
#undef LAL_WAIT_CASE
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;  // never looser than asked
  }
}

// This lane's index within the wavefront, from an instruction the compiler
// treats as having side effects, so values derived from it are computed where
// they are used instead of being kept live across loops.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl<0, N>(f);
}

template <int D, int DV, int NT>
struct Plan {
  static constexpr int CPRK = D / 8;   // 16-byte chunks per K row / state-copy row
  static constexpr int CPRV = DV / 8;  // per V-slice row
  static constexpr int NJ = DV / 16;
  static constexpr int NI = D / 16;
  static constexpr int NKC = D / 32;  // even: the Q rows load in pairs of steps
  static constexpr int BLKP = NT * 16;  // staged rows per block, a multiple of 32
  static constexpr int NCC = BLKP / 32;
  // phase A: RG row-tile pairs x CG column groups
  static constexpr int RG = NT / 2;
  static constexpr int CG0 = kWaves / RG;
  static constexpr int CG = CG0 < NJ ? CG0 : NJ;
  static constexpr int NJC = NJ / CG;
  // output stores per block and wave: pairs of value tiles are written
  // together, 16 bytes per lane (see store_o_pair), when a wave has an even
  // number of them
  static constexpr bool PAIR = NJC % 2 == 0;
  static constexpr bool QUAD = NJC % 4 == 0;  // whole 128-byte lines (store_o_quad)
  static constexpr int NST = PAIR ? NJC : 2 * NJC;            // store instructions
  static constexpr int NSTI = QUAD ? NJC / 2 : NST;            // store calls (a quad call issues 2)
  static constexpr int AWAVES = RG * CG;
  // phase B: PBR x PBC grid of waves over the state tiles
  static constexpr int PBR = kWaves < 4 ? kWaves : 4;
  static constexpr int PBC = kWaves / PBR;
  static constexpr int BIT = NI / PBR;
  static constexpr int BJT = NJ / PBC;
  // direct loads: 512 elements (1 KiB) per wave instruction
  static constexpr int KRPI = 512 / D;
  static constexpr int VRPI = 512 / DV;
  static constexpr int KINST = BLKP / KRPI;
  static constexpr int VINST = BLKP / VRPI;
  // Every wave issues the same number of direct loads per block (slots past
  // KINST / VINST load nothing and write zeros into rows past BLKP), so the
  // number of loads in flight is a compile-time constant.
  static constexpr int KI_W = (KINST + kWaves - 1) / kWaves;
  static constexpr int VI_W = (VINST + kWaves - 1) / kWaves;
  static constexpr int N_DMA = KI_W + VI_W;
  static_assert(KI_W * kWaves * KRPI <= kBlkMax && VI_W * kWaves * VRPI <= kBlkMax, "padding slots stay in the tile");
  static_assert(N_DMA <= 16, "vmcnt immediate");
  // Vector-memory issue slots of phase A: the NKC inter-block steps and the
  // first NCH_MIN key chunks (every row-tile pair has at least that many).
  static constexpr int NCH_MIN = (NT / 2) / 2 + 1;
  static constexpr int NSLOT = NKC + NCH_MIN;
  static_assert(NT % 2 == 0 && NT >= 2 && NT <= 8, "2..8 row tiles per block");
  static_assert(NKC % 2 == 0, "whole-line Q loads");
  static_assert(NJ % CG == 0 && AWAVES <= kWaves, "phase A grid");
  static_assert(BIT >= 1 && BJT >= 1, "phase B grid");
  static_assert(BLKP % KRPI == 0 && BLKP % VRPI == 0, "direct-load rows");
};

template <int D, int DV, int NT, int SM>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_bf16_kernel(PrefillArgs a) {
  using P = Plan<D, DV, NT>;
  // Two stages of K and V tiles, and the bf16 copy of the state slice.
  __shared__ __attribute__((aligned(1024))) u16 Ks0[kBlkMax * D];
  __shared__ __attribute__((aligned(1024))) u16 Ks1[kBlkMax * D];
  __shared__ __attribute__((aligned(1024))) u16 Vs0[kBlkMax * DV];
  __shared__ __attribute__((aligned(1024))) u16 Vs1[kBlkMax * DV];
  __shared__ __attribute__((aligned(1024))) u16 SsT[DV * D];  // SsT[j][i] = bf16(S[i][j0 + j])
  // One-launch parts with at most 64 value columns leave 48 KiB of LDS free:
  // there the Q rows of blocks 1 .. nblk-1 of a short part are staged
  // (QSLOT blocks), laid out and swizzled as K tiles.
  constexpr bool QLDS = SM == kPsPartLB && DV <= 64;
  constexpr int kQsElems = QLDS ? 48 * 1024 / 2 : 8;
  constexpr int QSLOT = QLDS ? kQsElems / (16 * NT * D) : 0;
  __shared__ __attribute__((aligned(1024))) u16 Qs[kQsElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is uniform across the wave; saying so lets every loop and
  // branch that depends on it run on the scalar unit.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (sequence, value slice).  With several slices per sequence
  // and a grid that is a multiple of 8 * nsplit, the slices of one sequence
  // get workgroup ids congruent mod 8, i.e. the same XCD (workgroups are
  // dispatched round-robin over the 8 XCDs), so their common Q and K reads
  // can hit that XCD's L2.
  const int nsplit = a.nsplit;
  int64_t bh;
  int split;
  const int64_t wg = blockIdx.x;
  if (nsplit > 1 && a.xcd_map) {
    const int64_t xcd = wg & 7, local = wg >> 3;
    split = (int)(local % nsplit);
    bh = (local / nsplit) * 8 + xcd;
  } else {
    bh = wg / nsplit;
    split = (int)(wg % nsplit);
  }
  // paired gradient passes: the slice index selects the pass, not columns
  constexpr bool PAIR_PASS = SM == kPsGradRevPair;
  const bool second = PAIR_PASS && split == 1;
  const int j0 = PAIR_PASS ? 0 : split * DV;
  const int64_t N = a.N;
  const int blk = a.blk;
  // Block bookkeeping in 32-bit scalars (the host guarantees N / blk < 2^31).
  const int nfull = (int)(N / blk);                       // blocks of blk tokens
  const int last = (int)(N - (int64_t)nfull * blk);       // tokens in a final partial block
  const int nblk = nfull + (last > 0 ? 1 : 0);
  constexpr bool REV = SM == kPsGradRev || SM == kPsGradRevPair || SM == kPsGradFused;
  constexpr bool FUSED = SM == kPsGradFused;
  constexpr bool NARROW = SM == kPsBF16 || SM == kPsE4M3;
  constexpr bool GRAD = SM >= kPsGrad && SM <= kPsGradFused;
  constexpr bool PART_LB = SM == kPsPartLB;
  constexpr bool PART = SM == kPsPart || PART_LB;
  // a part's sequence and its place in it (PART), else the sequence itself
  const int64_t pseq = PART ? bh / a.part_P : bh;
  const int ppart = PART ? (int)(bh % a.part_P) : 0;
  // one-launch parts: block 0's tiles and Q rows requested before the main
  // loop (lb_issued); every block's K and V tiles held in LDS from before the
  // main loop to its end, where they fit the staging ring (kv_res); the Q
  // rows of blocks 1 .. nblk-1 staged in LDS before the main loop too, where
  // they fit its Q slots (q_res)
  [[maybe_unused]] bool lb_issued = false, kv_res = false, q_res = false;
  // first token (memory order) of the block processed at step j, of length len
  auto blk_tok0 = [&](int j, int len) -> int64_t {
    if constexpr (REV)
      return len > 0 ? N - (int64_t)j * blk - len : 0;
    else
      return (int64_t)j * blk;
  };
  // state snapshots per sequence
  const int nsnap = (SM == kPsF32Snap && a.snap) ? nfull / a.snap_every : 0;

  const u16 *qh = (second ? a.q2 : a.q) + (size_t)bh * (size_t)N * D;
  const u16 *kh = (second ? a.k2 : a.k) + (size_t)bh * (size_t)N * D;
  const u16 *vh = (second ? a.v2 : a.v) + (size_t)bh * (size_t)N * D;  // slice offset j0 added per load
  u16 *oh = (second ? a.o2 : a.o) + (size_t)bh * (size_t)N * D + j0;
  // fused dK/dV: the second role's queries (v rows) and outputs (dk)
  const u16 *qh2 = FUSED ? a.q2 + (size_t)bh * (size_t)N * D : nullptr;
  u16 *oh2 = FUSED ? a.o2 + (size_t)bh * (size_t)N * D : nullptr;
  const float *g_in = second ? a.g_in2 : a.g_in;
  const int g_in_t = second ? a.g_in_t2 : a.g_in_t;
  float *g_out = second ? a.g_out2 : a.g_out;
  const size_t st0 = (size_t)bh * D * D + j0;  // this slice of the state (elements)

  constexpr int RB = D * 2;    // bytes per K row and per state-copy row
  constexpr int VRB = DV * 2;  // bytes per V-slice row

  // ---- phase B ownership: i-tiles [ib*BIT, +BIT) x j-tiles [jb*BJT, +BJT) ----
  const int ib = wave % P::PBR, jb = wave / P::PBR;
  // state element (x, y, e) of this lane: tile row ib*BIT+x, tile column
  // jb*BJT+y, row 4g+e and column lr inside the tile
  auto s_at = [&](int x, int y, int e) {
    return st0 + (size_t)((ib * P::BIT + x) * 16 + 4 * g + e) * D + (jb * P::BJT + y) * 16 + lr;
  };
  // narrow formats: stored value = code * scale
  float lp_sc = 1.f;
  if constexpr (NARROW) {
    if (a.lp_scale) lp_sc = a.lp_scale[bh];
  }
  const float lp_inv = 1.f / lp_sc;
  f32x4 S_acc[P::BIT][P::BJT];
#pragma unroll
  for (int x = 0; x < P::BIT; ++x)
#pragma unroll
    for (int y = 0; y < P::BJT; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (SM == kPsBF16)
          S_acc[x][y][e] = bf16_bits_to_f32(((const u16 *)a.lp_state)[s_at(x, y, e)]) * lp_sc;
        else if constexpr (SM == kPsE4M3)
          S_acc[x][y][e] = __builtin_amdgcn_cvt_f32_fp8((int)((const uint8_t *)a.lp_state)[s_at(x, y, e)], 0) * lp_sc;
        else if constexpr (PART_LB)
          S_acc[x][y][e] = 0.f;  // the part's own K^T V is summed first
        else if constexpr (PART)
          S_acc[x][y][e] = a.part_s0[(size_t)pseq * D * D + (s_at(x, y, e) - (size_t)bh * D * D)];
        else if constexpr (GRAD)
          S_acc[x][y][e] = !g_in ? 0.f
                           : g_in_t ? g_in[(size_t)bh * D * D +
                                           (size_t)(j0 + (jb * P::BJT + y) * 16 + lr) * D +
                                           (ib * P::BIT + x) * 16 + 4 * g + e]
                                    : g_in[s_at(x, y, e)];
        else
          S_acc[x][y][e] = a.state[s_at(x, y, e)];
      }

  // A part of a sequence cut along the tokens starts from S_0 plus the K^T V
  // sums of the parts before it, added in part order.  The lane's elements of
  // UNR consecutive sums are loaded before any of them is added (the sums are
  // independent loads), so the prologue pays one memory round trip per UNR
  // sums rather than one per sum.
  if constexpr (PART && !PART_LB) {
    constexpr int NE = P::BIT * P::BJT * 4;
    constexpr int UNR = NE <= 16 ? 8 : (NE <= 32 ? 4 : 2);
    const int nsum = ppart * a.part_S;
    for (int c0 = 0; c0 < nsum; c0 += UNR) {
      float t[UNR][P::BIT][P::BJT][4];
#pragma unroll
      for (int i = 0; i < UNR; ++i) {
        const int c = c0 + i < nsum ? c0 + i : nsum - 1;
        const float *ps = a.part_sums + ((size_t)c * a.part_BH + (size_t)pseq) * D * D - (size_t)bh * D * D;
#pragma unroll
        for (int x = 0; x < P::BIT; ++x)
#pragma unroll
          for (int y = 0; y < P::BJT; ++y)
#pragma unroll
            for (int e = 0; e < 4; ++e) t[i][x][y][e] = ps[s_at(x, y, e)];
      }
#pragma unroll
      for (int i = 0; i < UNR; ++i)
#pragma unroll
        for (int x = 0; x < P::BIT; ++x)
#pragma unroll
          for (int y = 0; y < P::BJT; ++y)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c0 + i < nsum) S_acc[x][y][e] += t[i][x][y][e];
    }
  }

  // ---- phase A role: row tiles {rg, NT-1-rg} x value tiles [jc0, jc0 + NJC) ----
  const bool act = P::AWAVES == kWaves || wave < P::AWAVES;
  const int rg = wave % P::RG;
  const int jc0 = (wave / P::RG) * P::NJC;

  // ---- per-lane LDS byte offsets ----
  // Every tile row used below is a multiple of 16 plus a lane-dependent part,
  // and the swizzle only looks at the low 4 row bits, so each access is a
  // per-lane part plus a compile-time row offset (an immediate).  The
  // per-lane parts are recomputed (a few integer operations) from a lane id
  // the compiler cannot hoist, where they are used: keeping all of them live
  // across the block loop would cost ~40 registers the matrix pipeline needs.
  struct LaneOff {
    int lr, g, h, lo8, rr;
  };
  auto lane_off = [&]() __attribute__((always_inline)) {
    const int ln = lane_now();
    LaneOff o;
    o.lr = ln & 15;
    o.g = ln >> 4;
    o.h = (o.lr & 3) >> 1;
    o.lo8 = 8 * (o.lr & 1);
    o.rr = 4 * o.g + (o.lr >> 2);  // row of a transposing read within 16
    return o;
  };
  // 16-byte fragment of row lr for contraction step kc (K rows and the state
  // copy).  Step kc takes from 128-byte line kc/2 of the row the chunks of
  // parity kc%2, chunk 2g + kc%2 for lane group g, rather than four adjacent
  // chunks: the contraction over the head dimension may run in any order
  // that all its operands share, and in this one the Q rows load as whole
  // lines (see load_q_part).
  auto kfrag = [&](const LaneOff &o, int kc) {
    return o.lr * RB + (swz<P::CPRK>(o.lr, 8 * (kc >> 1) + 2 * o.g + (kc & 1)) << 4);
  };
  // transposing-read operand of value tile jt (V) and key tile it (K^T)
  auto vtr = [&](const LaneOff &o, int jt) { return o.rr * VRB + (swz<P::CPRV>(o.rr, 2 * jt + o.h) << 4) + o.lo8; };
  auto ktr = [&](const LaneOff &o, int it) { return o.rr * RB + (swz<P::CPRK>(o.rr, 2 * it + o.h) << 4) + o.lo8; };

  auto ld128 = [](const u16 *base, int off) { return *(const bf16x8 *)((const char *)base + off); };
  auto ldtr = [](const u16 *base, int off0, int off1) {
    return join_tr(lds_read_tr((const u16 *)((const char *)base + off0)),
                   lds_read_tr((const u16 *)((const char *)base + off1)));
  };

  auto write_state_copy = [&]() {
    const LaneOff lo = lane_off();
    const int lr = lo.lr, g = lo.g;
#pragma unroll
    for (int x = 0; x < P::BIT; ++x)
#pragma unroll
      for (int y = 0; y < P::BJT; ++y) {
        const int off = ((jb * P::BJT + y) * 16 + lr) * RB + (swz<P::CPRK>(lr, 2 * (ib * P::BIT + x) + (g >> 1)) << 4) +
                        8 * (g & 1);
        lds_store_b64((const char *)SsT + off, pack_bf16x4(S_acc[x][y]));
      }
  };

  // Per-lane parts of the Q-row load and output-store offsets (bytes),
  // computed once.  A Q-row load gives lane (lr, g) row r = lr mod 8 (+ 8 h)
  // of a row tile and 16 bytes at element 16 g + 8 (lr / 8) of a 128-byte
  // line; a quad store gives it token lr mod 8 (+ 8 h) and bytes
  // 64 (lr / 8) + 16 g of a 128-byte piece.  Reversed order puts row r of a
  // block at len - 1 - r: the per-lane part is then -r D.
  const int q_lane = [&] {
    const LaneOff lo = lane_off();
    const int col = 16 * lo.g + 8 * (lo.lr >> 3);
    return ((REV ? -(lo.lr & 7) : (lo.lr & 7)) * D + col) * 2;
  }();
  const int st_lane = [&] {
    const LaneOff lo = lane_off();
    return (REV ? -(lo.lr & 7) : (lo.lr & 7)) * D * 2 + (lo.lr >> 3) * 64 + 16 * lo.g;
  }();

  // ---- Q rows of the wave's two row tiles (registers) ----
  bf16x8 bq[2][P::NKC], qn[2][P::NKC];
  bf16x8 qv[2][P::NKC];  // fused dK/dV: the block's v rows (the dK role's queries)
  // Row tiles of the wave's pair: T0 = rg and T1 = NT-1-rg.  Waves without
  // phase-A work load and store nothing through zero-size descriptors, so
  // that every wave issues the same vector-memory operations.
  const int T0 = rg, T1 = NT - 1 - rg;
  // (cache policy 2: non-temporal, as the K/V tiles -- Q rows are read once)
  // Load m = 2l + h of row tile u reads rows 8h..8h+7 of the tile, 128-byte
  // line l of each: lane (lr, g) takes row 8h + (lr & 7), chunk 2g + (lr >> 3)
  // of the line.  Each row's line is read by one instruction, so the L1 sends
  // it to L2 as one 128-byte request; the operand fragments are rearranged
  // from these registers at the start of the block that uses them (take_q).
  // (vrows: the fused kernel's v rows into qv, else the query rows into qn)
  auto load_q_part = [&](int64_t tok0, int len, int u, int m, bool vrows = false) __attribute__((always_inline)) {
    // descriptor built from scalar-forced words: with the generic builder the
    // compiler could not prove it uniform and looped over lanes per load
    const u32x4 dq = raw_desc((vrows ? qh2 : qh) + (size_t)tok0 * D, act ? (uint32_t)len * D * 2 : 0u);
    __amdgpu_buffer_rsrc_t rq;
    __builtin_memcpy(&rq, &dq, sizeof(rq));
    const int l = m >> 1, h = m & 1;
    if constexpr (REV) {
      // row 16 T + r is token len-1-16T-r of the span (negative: padding)
      const int qoff = q_lane + (len - 1 - 16 * (u ? T1 : T0) - 8 * h) * D * 2;
      const bf16x8 x = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rq, qoff, l * 128, 2));
      if (vrows)
        qv[u][m] = x;
      else
        qn[u][m] = x;
    } else {
      qn[u][m] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               rq, q_lane, ((16 * (u ? T1 : T0) + 8 * h) * D + 64 * l) * 2, 2));
    }
  };
  // Operand fragments from the loaded lines.  Step 2l (chunk 2g of line l for
  // lane group g) is, for rows lr < 8, what load 2l holds in the same lane
  // and, for rows 8..15, what load 2l+1 holds in lane lr ^ 8; step 2l+1 the
  // other way round.  A row rotation by 8 (DPP row_ror:8) written only to the
  // lanes of the upper (bank mask 0xc) or the lower (0x3) half of each row
  // does each in one move per dword.
  auto take_q = [&](bool vrows = false) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int l = 0; l < P::NKC / 2; ++l) {
        const u32x4 a = __builtin_bit_cast(u32x4, vrows ? qv[u][2 * l] : qn[u][2 * l]);
        const u32x4 b = __builtin_bit_cast(u32x4, vrows ? qv[u][2 * l + 1] : qn[u][2 * l + 1]);
        u32x4 e, o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          e[w] = (uint32_t)__builtin_amdgcn_update_dpp((int)a[w], (int)b[w], 0x128 /* row_ror:8 */, 0xf, 0xc, false);
          o[w] = (uint32_t)__builtin_amdgcn_update_dpp((int)b[w], (int)a[w], 0x128 /* row_ror:8 */, 0xf, 0x3, false);
        }
        bq[u][2 * l] = __builtin_bit_cast(bf16x8, e);
        bq[u][2 * l + 1] = __builtin_bit_cast(bf16x8, o);
      }
  };
  auto load_q = [&](int64_t tok0, int len) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kc = 0; kc < P::NKC; ++kc) load_q_part(tok0, len, u, kc);
  };

  // ---- direct HBM -> LDS loads of the K and V tiles of one block ----
  // Rows past len (a partial last block) and the padding slots read zeros.
  // A wave issues N_DMA such loads per block, one at a time (kv_issue), so
  // that they can be spread over the matrix work of the previous block.
  struct KvDma {
    int64_t tok0;
    int len;
    unsigned kl, vl;  // LDS byte addresses of the destination K and V tiles
  };
  auto kv_prepare = [&](int64_t tok0, int len, u16 *Kd, u16 *Vd) __attribute__((always_inline)) {
    return KvDma{tok0, len, lds_addr(Kd), lds_addr(Vd)};
  };
  // Per-lane part of the direct loads' byte offsets, computed once.  Load m
  // of a wave covers rows r0 + m kWaves RPI, r0 = wave RPI + lane / CPR;
  // kWaves RPI is a multiple of 16 and the swizzle of a row depends on the
  // row mod 16 only, so every load's offset is this part plus a uniform step.
  // Reversed order reads row r at (len - 1 - r) RB: the per-lane part is then
  // -r0 RB (rows past the block get negative offsets, outside the buffer).
  const int kv_lk = [&] {
    const int ln = lane_now();
    const int r0 = wave * P::KRPI + ln / P::CPRK;
    return (REV ? -r0 : r0) * RB + (swz<P::CPRK>(r0, ln % P::CPRK) << 4);
  }();
  const int kv_lv = [&] {
    const int ln = lane_now();
    const int r0 = wave * P::VRPI + ln / P::CPRV;
    return (REV ? -r0 : r0) * RB + (swz<P::CPRV>(r0, ln % P::CPRV) << 4) + j0 * 2;
  }();
  // The descriptors are rebuilt for every load (a few scalar operations) so
  // that none of them occupies scalar registers across the matrix work.
  auto kv_issue = [&](const KvDma &d, int m) __attribute__((always_inline)) {
    unsigned zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    const bool is_k = m < P::KI_W;
    const int mm = is_k ? m : m - P::KI_W;
    const int inst = wave + kWaves * mm;
    const int step = mm * kWaves * (is_k ? P::KRPI : P::VRPI) * RB;  // bytes
    const int off = (is_k ? kv_lk : kv_lv) + (REV ? (d.len - 1) * RB - step : step);
    const u32x4 desc = raw_desc((is_k ? kh : vh) + (size_t)d.tok0 * D,
                                inst < (is_k ? P::KINST : P::VINST) ? (uint32_t)d.len * D * 2 + zero : 0u);
    const unsigned lds = (is_k ? d.kl : d.vl) + inst * 1024;  // 512 elements per load
    if constexpr (PAIR_PASS)
      dma_b128_shared(desc, off, lds);
    else
      dma_b128(desc, off, lds);
  };
  auto kv_issue_all = [&](const KvDma &d) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < P::N_DMA; ++m) kv_issue(d, m);
  };
  // Q rows of block b >= 1 into its LDS slot (one-launch parts, QLDS), by
  // the K tiles' direct loads
  [[maybe_unused]] auto q_slot = [&](int b) { return Qs + (b - 1) * 16 * NT * D; };
  [[maybe_unused]] auto q_issue = [&](int64_t tok0, int len, u16 *Qd) __attribute__((always_inline)) {
    unsigned zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
#pragma unroll
    for (int m = 0; m < P::KI_W; ++m) {
      const int inst = wave + kWaves * m;
      const int step = m * kWaves * P::KRPI * RB;
      const u32x4 desc = raw_desc(qh + (size_t)tok0 * D, inst < P::KINST ? (uint32_t)len * D * 2 + zero : 0u);
      dma_b128(desc, kv_lk + step, lds_addr(Qd) + inst * 1024);
    }
  };
  auto block_len = [&](int jb) { return jb < nfull ? blk : last; };


  // ---- phase A for row-tile pair {RGI, NT-1-RGI}: output rows ----
  // (tstate: read the state copy transposed, for the fused kernel's dK role)
  auto phase_a = [&](auto rgi, const u16 *Kc, const u16 *Vc, f32x4 (&acc)[2][P::NJC], auto &&vm_slot,
                     auto tstate) __attribute__((always_inline)) {
    constexpr bool TS = decltype(tstate)::value;

    constexpr int T[2] = {decltype(rgi)::value, NT - 1 - decltype(rgi)::value};
    constexpr int NCH = T[1] / 2 + 1;  // 32-key chunks this pair touches

    // Operands of a 32-key chunk: K rows (A operand of P^T = K Q^T, one
    // buffer, refilled for the next chunk as soon as this chunk's P products
    // have been issued) and V^T (A operand of O^T += V^T P^T, two buffers).
    auto need = [](int cc, int s, int u) constexpr { return 2 * cc + s <= T[u] && cc <= T[u] / 2; };
    const LaneOff lo = lane_off();
    int kf[P::NKC], vtrA[P::NJC];
#pragma unroll
    for (int kc = 0; kc < P::NKC; ++kc) kf[kc] = kfrag(lo, kc);
#pragma unroll
    for (int jl = 0; jl < P::NJC; ++jl) vtrA[jl] = vtr(lo, jc0 + jl);
    bf16x8 kbuf[2][P::NKC];
    bf16x8 vbuf[2][P::NJC];
    auto load_k = [&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (!need(cc, s, 0) && !need(cc, s, 1)) continue;
#pragma unroll
        for (int kc = 0; kc < P::NKC; ++kc) kbuf[s][kc] = ld128(Kc, kf[kc] + (32 * cc + 16 * s) * RB);
      }
    };
    auto load_v = [&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
      const int c0 = 32 * cc;
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl)
        vbuf[cc & 1][jl] = ldtr(Vc, vtrA[jl] + c0 * VRB, vtrA[jl] + (c0 + 16) * VRB);
    };

    // inter-block part: O^T += S^T Q^T (each state operand feeds both row
    // tiles).  The state operands of step kc + 1 are requested before the
    // products of step kc; the first key chunk's operands during the last two.
    bf16x8 sfr[P::NKC][P::NJC];
    auto load_s = [&](int kc) __attribute__((always_inline)) {
      if constexpr (TS) {
        // A = S itself: lane (i, g) needs S[16 (jc0 + jl) + i][8 tau + e],
        // tau = 8 (kc / 2) + 2 g + kc % 2 (the head-dimension order of the
        // query fragments), i.e. column 16 (jc0 + jl) + i of rows
        // 8 tau + e of the copy: two transposing reads whose 16 lanes
        // address rows 8 tau + lr / 4 (+ 4) and columns + 4 (lr % 4).  The
        // lane's rows and its swizzle bits are formed once per step: a
        // row's swizzle is an XOR with bits of the row mod 16, and the
        // value tiles only change the logical chunk's upper bits.
        const LaneOff lt = lane_off();
        const int r0 = 8 * (8 * (kc >> 1) + 2 * lt.g + (kc & 1)) + (lt.lr >> 2), r1 = r0 + 4;
        const int b0 = r0 * RB + lt.lo8, b1 = r1 * RB + lt.lo8;
        const int x0 = swz<P::CPRK>(r0, lt.h) << 4, x1 = swz<P::CPRK>(r1, lt.h) << 4;
#pragma unroll
        for (int jl = 0; jl < P::NJC; ++jl)
          sfr[kc][jl] = ldtr(SsT, b0 + ((32 * (jc0 + jl)) ^ x0), b1 + ((32 * (jc0 + jl)) ^ x1));
      } else {
#pragma unroll
        for (int jl = 0; jl < P::NJC; ++jl) sfr[kc][jl] = ld128(SsT, kf[kc] + (jc0 + jl) * 16 * RB);
      }
    };
    load_s(0);
#pragma unroll
    for (int kc = 0; kc < P::NKC; ++kc) {
      vm_slot(kc);  // a share of the next block's Q rows and K/V tiles
      if (kc + 1 < P::NKC) load_s(kc + 1);
      if (kc == P::NKC - 2 || (P::NKC == 1 && kc == 0)) load_k(std::integral_constant<int, 0>{});
      if (kc == P::NKC - 1) load_v(std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) {
        acc[0][jl] = mfma_16x16x32(sfr[kc][jl], bq[0][kc], acc[0][jl]);
        acc[1][jl] = mfma_16x16x32(sfr[kc][jl], bq[1][kc], acc[1][jl]);
      }
    }

    // intra-block part, 32 keys at a time: O^T += V^T (P ⊙ M)^T.  Chunk cc
    // holds keys 32cc .. 32cc+31; row tile t uses chunks 0 .. t/2, and only
    // its last chunk straddles the diagonal.
    static_for<NCH>([&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (cc < P::NCH_MIN) vm_slot(P::NKC + cc);
      // pt[u][s][e] = P[16 T_u + lr][32 cc + 16 s + 4g + e]   (P^T = K Q^T)
      f32x4 pt[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          pt[u][s] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (!need(cc, s, u)) continue;
#pragma unroll
          for (int kc = 0; kc < P::NKC; ++kc) pt[u][s] = mfma_16x16x32(kbuf[s][kc], bq[u][kc], pt[u][s]);
        }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (cc + 1 < NCH) {
        load_k(std::integral_constant<int, cc + 1>{});
        load_v(std::integral_constant<int, cc + 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (cc > T[u] / 2) continue;
        // keys 16(2cc+s) + 4g + e against token 16 T_u + lr
        bf16x8 pb;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kt = 2 * cc + s;  // 16-key tile index
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bf16 val;
            if (kt < T[u])
              val = (bf16)pt[u][s][e];  // whole tile below the diagonal
            else if (kt == T[u])
              val = (4 * g + e <= lr) ? (bf16)pt[u][s][e] : (bf16)0.f;  // diagonal tile
            else
              val = (bf16)0.f;  // above the diagonal
            pb[4 * s + e] = val;
          }
        }
#pragma unroll
        for (int jl = 0; jl < P::NJC; ++jl) acc[u][jl] = mfma_16x16x32(vbuf[cc & 1][jl], pb, acc[u][jl]);
      }
    });

  };

  // Call f(integral_constant<int, rg>) for the wave's row-tile pair.
  // Exactly one call on every path (the last case is unconditional), which
  // lets the compiler count the memory operations each path issues.
  auto with_rg = [&](auto &&f) __attribute__((always_inline)) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, (P::RG > 1 ? 1 : 0)>;
    using I2 = std::integral_constant<int, (P::RG > 2 ? 2 : 0)>;
    using I3 = std::integral_constant<int, (P::RG > 3 ? 3 : 0)>;
    if constexpr (P::RG == 1) {
      f(I0{});
    } else if constexpr (P::RG == 2) {
      if (rg == 0) f(I0{}); else f(I1{});
    } else if constexpr (P::RG == 3) {
      if (rg == 0) f(I0{}); else if (rg == 1) f(I1{}); else f(I2{});
    } else {
      if (rg == 0) f(I0{}); else if (rg == 1) f(I1{}); else if (rg == 2) f(I2{}); else f(I3{});
    }
  };

  // ---- output rows of the wave's pair: acc[u][jl][e] =
  // O[16 T_u + lr][(jc0 + jl) * 16 + 4g + e].  Rows past len fall outside the
  // descriptor and are dropped, so every wave issues the same stores. ----
  auto store_o_part = [&](u16 *obase, int64_t tok0, int len, const uint2 (&packed)[2][P::NJC], int u, int jl)
                          __attribute__((always_inline)) {
    const u32x4 dod = raw_desc(obase + (size_t)tok0 * D, act ? (uint32_t)(len * D - j0) * 2 : 0u);
    __amdgpu_buffer_rsrc_t ro;
    __builtin_memcpy(&ro, &dod, sizeof(ro));
    // The row-tile part of the offset goes in the scalar offset, so each
    // lane needs one address register for all of these stores.
    const LaneOff lo_st = lane_off();
    if constexpr (REV) {
      const int orow = len - 1 - 16 * (u ? T1 : T0) - lo_st.lr;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, packed[u][jl]), ro,
                                            (orow * D + jc0 * 16 + 4 * lo_st.g) * 2 + jl * 32, 0, kStNT);
    } else {
      const int olane = (lo_st.lr * D + jc0 * 16 + 4 * lo_st.g) * 2;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, packed[u][jl]), ro, olane + jl * 32,
                                            16 * (u ? T1 : T0) * D * 2, kStNT);
    }
  };

  // Value tiles 2 jp and 2 jp + 1 of row tile u in one store.  In the
  // matrix-core output layout lane (lr, g) holds 4 consecutive values (8
  // bytes) of token 16 T_u + lr in each tile, so an output row would be
  // written in 32-byte pieces.  Two lane swaps across the four 16-lane rows
  // (the upper 32 lanes of one tile with the lower 32 of the other, then the
  // odd rows of one with the even rows of the other) leave lane (lr, g) with
  // values 8 g .. 8 g + 7 of the pair (16 bytes), so each row of the pair is
  // written as 64 contiguous bytes: half the store instructions, and half
  // the write requests, each holding an L1 slot.
  auto store_o_pair = [&](u16 *obase, int64_t tok0, int len, const uint2 (&packed)[2][P::NJC], int u, int jp)
                          __attribute__((always_inline)) {
    const u32x4 dod = raw_desc(obase + (size_t)tok0 * D, act ? (uint32_t)(len * D - j0) * 2 : 0u);
    __amdgpu_buffer_rsrc_t ro;
    __builtin_memcpy(&ro, &dod, sizeof(ro));
    const uint2 ta = packed[u][2 * jp], tb = packed[u][2 * jp + 1];
    const auto x1 = __builtin_amdgcn_permlane32_swap(ta.x, tb.x, false, false);
    const auto y1 = __builtin_amdgcn_permlane32_swap(ta.y, tb.y, false, false);
    const auto x2 = __builtin_amdgcn_permlane16_swap(x1[0], x1[1], false, false);
    const auto y2 = __builtin_amdgcn_permlane16_swap(y1[0], y1[1], false, false);
    const u32x4 data = {x2[0], y2[0], x2[1], y2[1]};
    const LaneOff lo_st = lane_off();
    if constexpr (REV) {
      const int orow = len - 1 - 16 * (u ? T1 : T0) - lo_st.lr;
      __builtin_amdgcn_raw_buffer_store_b128(data, ro, (orow * D + jc0 * 16) * 2 + 16 * lo_st.g + jp * 64, 0, kStNT);
    } else {
      const int olane = (lo_st.lr * D + jc0 * 16) * 2 + 16 * lo_st.g;
      __builtin_amdgcn_raw_buffer_store_b128(data, ro, olane + jp * 64, 16 * (u ? T1 : T0) * D * 2, kStNT);
    }
  };

  // Value tiles 4 jq .. 4 jq + 3 of row tile u in two stores that each write
  // 128 contiguous bytes -- one whole line -- for 8 of the 16 tokens.  After
  // the pair rearrangement of store_o_pair, lane (lr, g) holds 16 bytes of
  // pair A (tiles 4 jq, 4 jq + 1; bytes 0..63 of its token's span) and of pair
  // B (bytes 64..127).  Lanes lr and lr ^ 8 of a 16-lane row then trade one of
  // them (a rotation by 8 within the row): store h writes tokens 8 h .. 8 h + 7,
  // the lanes lr < 8 holding bytes 0..63 and the lanes lr >= 8 bytes 64..127.
  auto store_o_quad = [&](u16 *obase, int64_t tok0, int len, const uint2 (&packed)[2][P::NJC], int u, int jq)
                          __attribute__((always_inline)) {
    const u32x4 dod = raw_desc(obase + (size_t)tok0 * D, act ? (uint32_t)(len * D - j0) * 2 : 0u);
    __amdgpu_buffer_rsrc_t ro;
    __builtin_memcpy(&ro, &dod, sizeof(ro));
    u32x4 pr[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint2 ta = packed[u][4 * jq + 2 * h], tb = packed[u][4 * jq + 2 * h + 1];
      const auto x1 = __builtin_amdgcn_permlane32_swap(ta.x, tb.x, false, false);
      const auto y1 = __builtin_amdgcn_permlane32_swap(ta.y, tb.y, false, false);
      const auto x2 = __builtin_amdgcn_permlane16_swap(x1[0], x1[1], false, false);
      const auto y2 = __builtin_amdgcn_permlane16_swap(y1[0], y1[1], false, false);
      pr[h] = u32x4{x2[0], y2[0], x2[1], y2[1]};
    }
    const bool upper = (lane_now() & 15) >= 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // store h: the lower lanes keep pair A (h = 0) or take the partner's
      // pair A (h = 1); the upper lanes take the partner's pair B (h = 0) or
      // keep their own (h = 1)
      u32x4 data;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int moved = __builtin_amdgcn_update_dpp(0, (int)pr[1 - h][w], 0x128 /* row_ror:8 */, 0xf, 0xf, false);
        data[w] = (upper == (h == 0)) ? (uint32_t)moved : pr[h][w];
      }
      // token 8 h + lr mod 8 of the row tile, bytes 64 (lr / 8) + 16 g of
      // piece jq of the slice row
      const int cst = (jc0 * 16) * 2 + jq * 128;
      if constexpr (REV) {
        __builtin_amdgcn_raw_buffer_store_b128(data, ro, st_lane + (len - 1 - 16 * (u ? T1 : T0) - 8 * h) * D * 2 + cst,
                                               0, kStNT);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(data, ro, st_lane + 8 * h * D * 2 + cst, 16 * (u ? T1 : T0) * D * 2,
                                               kStNT);
      }
    }
  };

  // ---- a ring of block slots over both stages (one-launch parts): each
  // stage holds kBlkMax / (16 NT) blocks; the ring has at most 64 / N_DMA
  // slots so that every wait on the blocks in flight fits a vmcnt ----
  constexpr int NSUB = kBlkMax / (16 * NT);
  constexpr int RING = (2 * NSUB - 1) * P::N_DMA <= 63 ? 2 * NSUB : 63 / P::N_DMA + 1;
  [[maybe_unused]] auto slot_k = [&](int sl) { return (sl / NSUB ? Ks1 : Ks0) + (sl % NSUB) * 16 * NT * D; };
  [[maybe_unused]] auto slot_v = [&](int sl) { return (sl / NSUB ? Vs1 : Vs0) + (sl % NSUB) * 16 * NT * DV; };

  // ---- one block.  On entry the Q rows and direct loads of block jblk
  // (into Kc, Vc), then the output stores of block jblk-1, may be in flight;
  // the other stage (Kn, Vn) is free (its block's reads ended at the previous
  // block's second barrier).  During the block the wave issues the Q rows of
  // block jblk+1 (at the start), its K/V tiles (spread over the matrix work
  // of phase A, so that no burst stalls the wave on a full memory queue) and
  // this block's output stores (spread over phase B). ----
  auto body = [&](int jblk, const u16 *Kc, const u16 *Vc, u16 *Kn, u16 *Vn) __attribute__((always_inline)) {
    // (in forward order the reversed arms fold away at compile time, leaving
    // exactly the forward kernel's code)
    const int64_t tok0 = REV ? blk_tok0(jblk, block_len(jblk)) : (int64_t)jblk * blk;
    const int len = block_len(jblk);
    const int nlen = jblk + 1 < nblk ? block_len(jblk + 1) : 0;
    // Wait for this block's tiles and Q rows; the previous block's 2 NJC
    // output stores, issued after them, may stay in flight.
    wait_vmcnt(jblk == 0 ? 0 : P::NST);
    if (PART_LB && q_res && jblk > 0) {
      // Q rows from their LDS slot, in the fragment order of the K rows
      // (filled before the main loop; block 0's wait and barrier made them
      // visible)
      const LaneOff lq = lane_off();
      const u16 *Qc = q_slot(jblk);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kc = 0; kc < P::NKC; ++kc) bq[u][kc] = ld128(Qc, kfrag(lq, kc) + 16 * (u ? T1 : T0) * RB);
    } else {
      take_q();
    }
    lds_barrier();  // every wave's tiles of block jblk and the state copy are in LDS

    // the next block's loads, one share per issue slot
    const KvDma dma = kv_prepare(REV ? blk_tok0(jblk + 1, nlen) : tok0 + blk, nlen, Kn, Vn);
    // The next block's Q rows, issued here in code that every wave runs: issued
    // inside the per-row-tile branches of phase A, their destination registers
    // differ between branches, and the compiler's wait analysis, which merges
    // the branches, then drains all loads in flight at the start of phase A.
    if (!(PART_LB && q_res)) {
#pragma unroll
      for (int kc = 0; kc < P::NKC; ++kc) {
        load_q_part(REV ? blk_tok0(jblk + 1, nlen) : tok0 + blk, nlen, 0, kc);
        load_q_part(REV ? blk_tok0(jblk + 1, nlen) : tok0 + blk, nlen, 1, kc);
      }
    }
    auto vm_slot = [&](int slot) __attribute__((always_inline)) {
      if (nlen > 0 && !(PART_LB && kv_res)) {
#pragma unroll
        for (int m = slot * P::N_DMA / P::NSLOT; m < (slot + 1) * P::N_DMA / P::NSLOT; ++m) kv_issue(dma, m);
      }
    };

    // ---------------- phase A: output rows ----------------
    f32x4 acc[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) acc[u][jl] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (act) {
      with_rg([&](auto rgi) { phase_a(rgi, Kc, Vc, acc, vm_slot, std::false_type{}); });
    } else {
#pragma unroll
      for (int slot = 0; slot < P::NSLOT; ++slot) vm_slot(slot);
    }
    uint2 packed[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) packed[u][jl] = pack_bf16x4(acc[u][jl]);

    // ---------------- phase B: state update S += K^T V ----------------
    // (with this block's output stores spread over its chunks)
    const LaneOff lob = lane_off();
    int ktrB[P::BIT], vtrB[P::BJT];  // K^T and V operands of phase B
#pragma unroll
    for (int x = 0; x < P::BIT; ++x) ktrB[x] = ktr(lob, ib * P::BIT + x);
#pragma unroll
    for (int y = 0; y < P::BJT; ++y) vtrB[y] = vtr(lob, jb * P::BJT + y);
#pragma unroll
    for (int cc = 0; cc < P::NCC; ++cc) {
      const int c0 = 32 * cc;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = cc * P::NSTI / P::NCC; i < (cc + 1) * P::NSTI / P::NCC; ++i) {
        if constexpr (P::QUAD)
          store_o_quad(oh, tok0, len, packed, i / (P::NJC / 4), i % (P::NJC / 4));
        else if constexpr (P::PAIR)
          store_o_pair(oh, tok0, len, packed, i / (P::NJC / 2), i % (P::NJC / 2));
        else
          store_o_part(oh, tok0, len, packed, i / P::NJC, i % P::NJC);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 ka[P::BIT], vb[P::BJT];
#pragma unroll
      for (int x = 0; x < P::BIT; ++x) ka[x] = ldtr(Kc, ktrB[x] + c0 * RB, ktrB[x] + (c0 + 16) * RB);
#pragma unroll
      for (int y = 0; y < P::BJT; ++y) vb[y] = ldtr(Vc, vtrB[y] + c0 * VRB, vtrB[y] + (c0 + 16) * VRB);
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y) S_acc[x][y] = mfma_16x16x32(ka[x], vb[y], S_acc[x][y]);
    }

    // the carry stored in the narrow format after every block (if asked)
    if constexpr (NARROW) {
      if (a.lp_round) {
#pragma unroll
        for (int x = 0; x < P::BIT; ++x)
#pragma unroll
          for (int y = 0; y < P::BJT; ++y) S_acc[x][y] = round_to_store<SM>(S_acc[x][y], lp_sc, lp_inv);
      }
    }

    // optional snapshot of S after this block (full blocks only)
    if (SM == kPsF32Snap && nsnap > 0 && (jblk + 1) % a.snap_every == 0 && (jblk + 1) / a.snap_every <= nsnap) {
      float *sp = a.snap + ((size_t)bh * nsnap + ((jblk + 1) / a.snap_every - 1)) * D * D + j0;
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sp[(size_t)((ib * P::BIT + x) * 16 + 4 * g + e) * D + (jb * P::BJT + y) * 16 + lr] = S_acc[x][y][e];
    }

    // Every wave's reads of this stage and of the state copy are complete
    // (only LDS accesses are drained, not the loads in flight).
    lds_barrier();
    write_state_copy();  // bf16 copy of S_jblk for the next block's phase A
  };

  // ---- one block of the fused dK/dV kernel (reversed order).  The stages
  // hold the block's q tile (Kc) and dout tile (Vc).  On entry the block's
  // tiles and k rows, then the previous block's dk stores, may be in flight.
  //  1. dV role: queries = k rows, keys = q, values = dout, state G as is;
  //  2. dK role: queries = v rows, keys = dout, values = q, state G^T;
  //  3. G += q^T dout.
  // The next block's k rows are issued at the start and its v rows between the
  // roles, in common code (each set is consumed one block later, so the
  // compiler's waits for them find every later load already counted); the
  // next block's tiles over both roles' issue slots, the dv stores over the
  // dK role's and the dk stores over step 3: memory work in every phase.
  auto body_fused = [&](int jblk, const u16 *Kc, const u16 *Vc, u16 *Kn, u16 *Vn) __attribute__((always_inline)) {
    const int64_t tok0 = blk_tok0(jblk, block_len(jblk));
    const int len = block_len(jblk);
    const int nlen = jblk + 1 < nblk ? block_len(jblk + 1) : 0;
    const int64_t ntok0 = blk_tok0(jblk + 1, nlen);
    wait_vmcnt(jblk == 0 ? 0 : P::NST);
    take_q();
    lds_barrier();
    const KvDma dma = kv_prepare(ntok0, nlen, Kn, Vn);
#pragma unroll
    for (int kc = 0; kc < P::NKC; ++kc) {
      load_q_part(ntok0, nlen, 0, kc);
      load_q_part(ntok0, nlen, 1, kc);
    }

    // 1. dV role, with the next block's tiles
    f32x4 acc[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) acc[u][jl] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the first half of the next block's direct loads over the dV role's
    // issue slots, the second half over the dK role's (reads in flight
    // through both roles)
    constexpr int NDH = P::N_DMA / 2;
    auto dma_slot = [&](int slot) __attribute__((always_inline)) {
      if (nlen > 0) {
#pragma unroll
        for (int m = slot * NDH / P::NSLOT; m < (slot + 1) * NDH / P::NSLOT; ++m) kv_issue(dma, m);
      }
    };
    if (act) {
      with_rg([&](auto rgi) { phase_a(rgi, Kc, Vc, acc, dma_slot, std::false_type{}); });
    } else {
#pragma unroll
      for (int slot = 0; slot < P::NSLOT; ++slot) dma_slot(slot);
    }
    uint2 packed_v[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) packed_v[u][jl] = pack_bf16x4(acc[u][jl]);

    // 2. dK role, with this block's dv stores; the next block's v rows first
    take_q(true);
#pragma unroll
    for (int kc = 0; kc < P::NKC; ++kc) {
      load_q_part(ntok0, nlen, 0, kc, true);
      load_q_part(ntok0, nlen, 1, kc, true);
    }
    auto vm_slot = [&](int slot) __attribute__((always_inline)) {
      if (nlen > 0) {
#pragma unroll
        for (int m = NDH + slot * (P::N_DMA - NDH) / P::NSLOT; m < NDH + (slot + 1) * (P::N_DMA - NDH) / P::NSLOT; ++m)
          kv_issue(dma, m);
      }
#pragma unroll
      for (int i = slot * P::NSTI / P::NSLOT; i < (slot + 1) * P::NSTI / P::NSLOT; ++i) {
        if constexpr (P::QUAD)
          store_o_quad(oh, tok0, len, packed_v, i / (P::NJC / 4), i % (P::NJC / 4));
        else if constexpr (P::PAIR)
          store_o_pair(oh, tok0, len, packed_v, i / (P::NJC / 2), i % (P::NJC / 2));
        else
          store_o_part(oh, tok0, len, packed_v, i / P::NJC, i % P::NJC);
      }
    };
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) acc[u][jl] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (act) {
      with_rg([&](auto rgi) { phase_a(rgi, Vc, Kc, acc, vm_slot, std::true_type{}); });
    } else {
#pragma unroll
      for (int slot = 0; slot < P::NSLOT; ++slot) vm_slot(slot);
    }
    uint2 packed_k[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) packed_k[u][jl] = pack_bf16x4(acc[u][jl]);

    // 3. G += q^T dout, with this block's dk stores
    const LaneOff lob = lane_off();
    int ktrB[P::BIT], vtrB[P::BJT];
#pragma unroll
    for (int x = 0; x < P::BIT; ++x) ktrB[x] = ktr(lob, ib * P::BIT + x);
#pragma unroll
    for (int y = 0; y < P::BJT; ++y) vtrB[y] = vtr(lob, jb * P::BJT + y);
#pragma unroll
    for (int cc = 0; cc < P::NCC; ++cc) {
      const int c0 = 32 * cc;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = cc * P::NSTI / P::NCC; i < (cc + 1) * P::NSTI / P::NCC; ++i) {
        if constexpr (P::QUAD)
          store_o_quad(oh2, tok0, len, packed_k, i / (P::NJC / 4), i % (P::NJC / 4));
        else if constexpr (P::PAIR)
          store_o_pair(oh2, tok0, len, packed_k, i / (P::NJC / 2), i % (P::NJC / 2));
        else
          store_o_part(oh2, tok0, len, packed_k, i / P::NJC, i % P::NJC);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 ka[P::BIT], vb[P::BJT];
#pragma unroll
      for (int x = 0; x < P::BIT; ++x) ka[x] = ldtr(Kc, ktrB[x] + c0 * RB, ktrB[x] + (c0 + 16) * RB);
#pragma unroll
      for (int y = 0; y < P::BJT; ++y) vb[y] = ldtr(Vc, vtrB[y] + c0 * VRB, vtrB[y] + (c0 + 16) * VRB);
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y) S_acc[x][y] = mfma_16x16x32(ka[x], vb[y], S_acc[x][y]);
    }
    lds_barrier();
    write_state_copy();
  };

  // ---- one-launch part (kPsPartLB): the part's start state ----
  // Flags of this sequence and value slice: published[j] and done[j] of part
  // j at pub[j * kPartMaxSplit] and done_f[j * kPartMaxSplit].  Every wait is
  // for a part of a lower workgroup id (parts are numbered along the grid in
  // order, for each slice), and a part publishes before it waits, so with
  // workgroups dispatched in id order every awaited part runs.
  // The sums and flags cross XCDs, whose L2 caches are not coherent with one
  // another.  They are written and read with device-scope (sc1) accesses,
  // which the L2 keeps coherent, rather than with acquire/release fences: a
  // device-scope fence writes back or invalidates the whole L2 of the XCD,
  // under the feet of the other workgroups streaming through it.  Order: a
  // part's sum stores complete (vmcnt) before any lane stores its flag; a
  // reader issues its sum loads only after its flag load has returned.
  [[maybe_unused]] unsigned long long *pub = nullptr, *slab_f = nullptr, *done_f = nullptr;
  auto flag_now = [&](const unsigned long long *f) __attribute__((always_inline)) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto wait_flag = [&](const unsigned long long *f) __attribute__((always_inline)) {
    bool seen = flag_now(f) == a.part_epoch;
    if (!seen) {
      const unsigned long long t0 = wall_clock64();
      do {
        __builtin_amdgcn_s_sleep(1);
        seen = flag_now(f) == a.part_epoch;
      } while (!seen && wall_clock64() - t0 < a.part_wait_ticks);
    }
    // later loads stay after the flag load (a compiler barrier; the flag's
    // value has returned before the loop ends)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return seen;
  };
  auto set_flag = [&](unsigned long long *f, unsigned long long v) __attribute__((always_inline)) {
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // whether v holds in any thread of the workgroup, through a word of the
  // state copy's LDS (every byte of LDS is taken; the copy is not in use
  // where this is called: before the main loop and after it)
  auto any_thread = [&](bool v) __attribute__((always_inline)) {
    __attribute__((address_space(3))) int *w = (__attribute__((address_space(3))) int *)(size_t)lds_addr(SsT);
    __syncthreads();
    if (tid == 0) *w = 0;
    __syncthreads();
    if (v) *w = 1;
    __syncthreads();
    const bool r = *w != 0;
    __syncthreads();
    return r;
  };
  // Sums and start states are stored in the order of the lanes' accumulator
  // fragments (part, sequence, slice: [wave][x][y][lane][4] floats), which
  // every workgroup of the slice shares, so that a lane moves 16 contiguous
  // bytes per access.  Steps of a part p (all parts of a sequence and slice
  // run them side by side):
  //  1. p < P-1: A_p = K^T V over its own tokens, published (flag pub[p]);
  //  2. every part takes 1/P of the slice's elements and forms, for them,
  //     the start of every part, start_{j+1} = start_j + A_j from start_0 =
  //     S_0, in part order; published (flag slab[p]);
  //  3. part p reads its own start (part 0: S_0) and sets done[p].
  // The last part stores S_N over S_0, and clears the flags, once every
  // other part is done.
  if constexpr (PART_LB) {
    const int np = a.part_P;
    pub = a.part_flags + (size_t)pseq * np * kPartMaxSplit + split;
    const size_t flag_stride = (size_t)a.part_BH * np * kPartMaxSplit;
    slab_f = pub + flag_stride;
    done_f = slab_f + flag_stride;
    // Byte offsets in the sums (and the starts, which follow them): element
    // (x, y) of this lane in region (j, seq, slice), and the region's base.
    // A one-launch cut has P <= kPartMaxOneLaunch and B H P <= the
    // compute-unit count, so both arrays span at most 2 (P - 1) B H d^2 4
    // < 2^31 bytes.
    const size_t region = (size_t)a.part_BH * D * D * 4;  // bytes from part j to j+1
    const uint32_t base0 = (uint32_t)(((size_t)pseq * D * D + (size_t)split * D * DV) * 4);
    const uint32_t lane0 = (uint32_t)(((size_t)wave * P::BIT * P::BJT * 256 + (size_t)lane_now() * 4) * 4);
    auto frag_at = [&](int j, int x, int y) {
      return base0 + lane0 + (uint32_t)((size_t)j * region + (size_t)(x * P::BJT + y) * 1024);
    };
    const uint32_t all_bytes = (uint32_t)(2 * (size_t)(np - 1) * region);
    const uint32_t starts0 = (uint32_t)((size_t)(np - 1) * region);
    const u32x4 dsum = raw_desc(a.part_sums_w, all_bytes);
    __amdgpu_buffer_rsrc_t rs;
    __builtin_memcpy(&rs, &dsum, sizeof(rs));
    // cache policy 16: sc1, device-scope coherent
    constexpr int kSc1 = 16;

    kv_res = nblk <= RING;
    if (ppart == np - 1 && kv_res) {
      // the last part has no sum to form: its tiles are requested now, into
      // the ring, and arrive while it waits for the other parts
      for (int b = 0; b < nblk; ++b) kv_issue_all(kv_prepare((int64_t)b * blk, block_len(b), slot_k(b), slot_v(b)));
    }
    if (ppart < np - 1) {
      // 1. K^T V over the part's own tokens (this slice's columns).  The
      // blocks' K and V tiles are staged as in the main loop, in the ring of
      // slots; where they all fit, they stay there for the main loop.
      const LaneOff lop = lane_off();
      int ktrP[P::BIT], vtrP[P::BJT];
#pragma unroll
      for (int x = 0; x < P::BIT; ++x) ktrP[x] = ktr(lop, ib * P::BIT + x);
#pragma unroll
      for (int y = 0; y < P::BJT; ++y) vtrP[y] = vtr(lop, jb * P::BJT + y);
      int issued = 0;
      for (; issued < nblk && issued < RING; ++issued)
        kv_issue_all(kv_prepare((int64_t)issued * blk, block_len(issued), slot_k(issued), slot_v(issued)));
      for (int pb = 0; pb < nblk; ++pb) {
        const int sl = pb % RING;
        const u16 *Kc = slot_k(sl);
        const u16 *Vc = slot_v(sl);
        wait_vmcnt((issued - pb - 1) * P::N_DMA);  // block pb has landed
        lds_barrier();
#pragma unroll
        for (int cc = 0; cc < P::NCC; ++cc) {
          const int c0 = 32 * cc;
          bf16x8 ka[P::BIT], vb[P::BJT];
#pragma unroll
          for (int x = 0; x < P::BIT; ++x) ka[x] = ldtr(Kc, ktrP[x] + c0 * RB, ktrP[x] + (c0 + 16) * RB);
#pragma unroll
          for (int y = 0; y < P::BJT; ++y) vb[y] = ldtr(Vc, vtrP[y] + c0 * VRB, vtrP[y] + (c0 + 16) * VRB);
#pragma unroll
          for (int x = 0; x < P::BIT; ++x)
#pragma unroll
            for (int y = 0; y < P::BJT; ++y) S_acc[x][y] = mfma_16x16x32(ka[x], vb[y], S_acc[x][y]);
        }
        lds_barrier();  // every wave is done with this slot
        if (issued < nblk) {
          kv_issue_all(kv_prepare((int64_t)issued * blk, block_len(issued), slot_k(sl), slot_v(sl)));
          ++issued;
        }
      }
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, S_acc[x][y]), rs, (int)frag_at(ppart, x, y), 0,
                                                 kSc1);
      wait_vmcnt(0);    // this wave's sum stores are complete
      __syncthreads();  // ... and every other wave's
      if (tid == 0) set_flag(pub + (size_t)ppart * kPartMaxSplit, a.part_epoch);
    }
    // the main loop's first tiles (unless held in the ring) and Q rows,
    // requested now so that they arrive during steps 2 and 3; the later
    // blocks' Q rows too, where they fit the Q slots
    {
      const int len0 = block_len(0);
      if (!kv_res) kv_issue_all(kv_prepare(0, len0, Ks0, Vs0));
      load_q(0, len0);
      if constexpr (QLDS) {
        q_res = kv_res && nblk - 1 <= QSLOT;
        if (q_res)
          for (int b = 1; b < nblk; ++b) q_issue((int64_t)b * blk, block_len(b), q_slot(b));
      }
      lb_issued = true;
    }

    // 2. the starts of every part for elements [ppart F, ppart F + F) of the
    // region (in float4s).  A thread's P - 1 sums are loaded together.
    bool ok = true;
    for (int j = tid; j < np - 1; j += kThreads)
      if (!wait_flag(pub + (size_t)j * kPartMaxSplit)) ok = false;
    // every sum is published, or some wait ran out: then the slab's starts are
    // NaN, so that no part starts from sums that were never written
    const bool sums_ok = !any_thread(!ok);
    {
      constexpr int E4 = D * DV / 4;
      const int F = E4 / np;
      for (int i = ppart * F + tid; i < (ppart + 1) * F; i += kThreads) {
        // fragment position -> state element: i = ((w BIT + x) BJT + y) 64 + l
        const int l = i & 63, t = i >> 6;
        const int y = t % P::BJT, x = (t / P::BJT) % P::BIT, w = t / (P::BJT * P::BIT);
        const int row = ((w % P::PBR) * P::BIT + x) * 16 + 4 * (l >> 4);
        const int col = j0 + ((w / P::PBR) * P::BJT + y) * 16 + (l & 15);
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = a.state[(size_t)pseq * D * D + (size_t)(row + e) * D + col];
        const uint32_t off = base0 + (uint32_t)i * 16;
        constexpr int kMaxTerms = kPartMaxOneLaunch - 1;
        f32x4 t4[kMaxTerms];
#pragma unroll
        for (int k = 0; k < kMaxTerms; ++k)
          if (k < np - 1)
            t4[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + k * region), 0, kSc1));
        if (!sums_ok) acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
        for (int k = 0; k < kMaxTerms; ++k)
          if (k < np - 1) {
            acc += t4[k];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), rs,
                                                   (int)(starts0 + off + k * region), 0, kSc1);
          }
      }
    }
    wait_vmcnt(0);  // this wave's start stores (and the tiles and Q rows above) are complete
    __syncthreads();
    if (tid == 0) set_flag(slab_f + (size_t)ppart * kPartMaxSplit, a.part_epoch);

    // 3. this part's start: S_0 for part 0, else start_p from every slab
    if (ppart == 0) {
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S_acc[x][y][e] = a.state[s_at(x, y, e) - (size_t)bh * D * D + (size_t)pseq * D * D];
    } else {
      for (int q = tid; q < np; q += kThreads)
        if (!wait_flag(slab_f + (size_t)q * kPartMaxSplit)) ok = false;
      __syncthreads();  // every slab is published
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y)
          S_acc[x][y] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(starts0 + frag_at(ppart - 1, x, y)), 0, kSc1));
    }
    // a wait that ran out (some part could not run): no valid start state
    if (any_thread(!ok)) {
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y)
          S_acc[x][y] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    if (ppart < np - 1) {
      // every wave has its start (the loads are consumed by the branch above)
#pragma unroll
      for (int x = 0; x < P::BIT; ++x)
#pragma unroll
        for (int y = 0; y < P::BJT; ++y) asm volatile("" ::"v"(S_acc[x][y]));
      __syncthreads();
      if (tid == 0) set_flag(done_f + (size_t)ppart * kPartMaxSplit, a.part_epoch);
    }
  }

  {
    const int len0 = block_len(0);
    if (!(PART_LB && lb_issued)) {
      kv_issue_all(kv_prepare(REV ? blk_tok0(0, len0) : 0, len0, Ks0, Vs0));
      load_q(REV ? blk_tok0(0, len0) : 0, len0);
    }
    if constexpr (FUSED) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kc = 0; kc < P::NKC; ++kc) load_q_part(blk_tok0(0, len0), len0, u, kc, true);
    }
    // The initial state and the first Q rows are consumed here, before the
    // loop, so the compiler's waits for their loads stay out of the
    // pipelined loop (where they would drain the loads in flight).
    write_state_copy();
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kc = 0; kc < P::NKC; ++kc) asm volatile("" ::"v"(qn[u][kc]));
    if constexpr (FUSED) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kc = 0; kc < P::NKC; ++kc) asm volatile("" ::"v"(qv[u][kc]));
    }
  }
  for (int jblk = 0; jblk < nblk; jblk += 2) {
    if constexpr (FUSED) {
      body_fused(jblk, Ks0, Vs0, Ks1, Vs1);
      if (jblk + 1 < nblk) body_fused(jblk + 1, Ks1, Vs1, Ks0, Vs0);
    } else if (PART_LB && kv_res) {
      // tiles held in the ring: no direct loads in the loop
      body(jblk, slot_k(jblk % RING), slot_v(jblk % RING), Ks0, Vs0);
      if (jblk + 1 < nblk) body(jblk + 1, slot_k((jblk + 1) % RING), slot_v((jblk + 1) % RING), Ks0, Vs0);
    } else {
      body(jblk, Ks0, Vs0, Ks1, Vs1);
      if (jblk + 1 < nblk) body(jblk + 1, Ks1, Vs1, Ks0, Vs0);
    }
  }

  // ---- final state ----
  // The last part of a one-launch cut stores S_N over S_0 only once every
  // other part of its slice has read S_0 (done flags).
  [[maybe_unused]] bool lb_done = true;
  if constexpr (PART_LB) {
    if (ppart == a.part_P - 1) {
      bool mine = true;
      for (int j = tid; j < a.part_P - 1; j += kThreads)
        if (!wait_flag(done_f + (size_t)j * kPartMaxSplit)) mine = false;
      lb_done = !any_thread(!mine);
    }
  }
  // Nothing of this wave may still be in flight when it ends: a gradient pass
  // may have no block to process, and then the first block's direct loads
  // into LDS were never awaited.  (Forward passes always have a block, whose
  // loads the loop awaits.)
  if constexpr (GRAD) wait_vmcnt(0);
#pragma unroll
  for (int x = 0; x < P::BIT; ++x)
#pragma unroll
    for (int y = 0; y < P::BJT; ++y) {
      if constexpr (SM == kPsE4M3) {
        const f32x4 sv = S_acc[x][y];
        const uint32_t w = f32_to_e4m3x4(f32x4{sv[0] * lp_inv, sv[1] * lp_inv, sv[2] * lp_inv, sv[3] * lp_inv});
#pragma unroll
        for (int e = 0; e < 4; ++e) ((uint8_t *)a.lp_state)[s_at(x, y, e)] = (uint8_t)(w >> (8 * e));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (SM == kPsBF16)
            ((u16 *)a.lp_state)[s_at(x, y, e)] = f32_to_bf16_bits(S_acc[x][y][e] * lp_inv);
          else if constexpr (GRAD) {
            if (g_out) g_out[s_at(x, y, e)] = S_acc[x][y][e];
          } else if constexpr (PART) {
            if (ppart == a.part_P - 1) a.state[(size_t)pseq * D * D + (s_at(x, y, e) - (size_t)bh * D * D)] = S_acc[x][y][e];
          } else
            a.state[s_at(x, y, e)] = S_acc[x][y][e];
        }
      }
    }
  // The last part of a one-launch cut then clears the flags of the other
  // parts (each is done with the flags and sums it reads), so that the next
  // call (or graph replay, with the same epoch) starts from zero.
  if constexpr (PART_LB) {
    if (ppart == a.part_P - 1 && lb_done) {
      for (int j = tid; j < a.part_P; j += kThreads) {
        if (j < a.part_P - 1) {
          set_flag(pub + (size_t)j * kPartMaxSplit, 0ull);
          set_flag(done_f + (size_t)j * kPartMaxSplit, 0ull);
        }
        set_flag(slab_f + (size_t)j * kPartMaxSplit, 0ull);
      }
    }
  }
}

template <int D, int DV, int SM>
hipError_t launch_nt(const PrefillArgs &a, int64_t BH, hipStream_t stream) {
  const int blkp = (a.blk + 31) & ~31;
  const dim3 grid((unsigned)(BH * a.nsplit)), block(kThreads);
  switch (blkp) {
    case 32: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 2, SM>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 4, SM>), grid, block, 0, stream, a); break;
    case 96: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 6, SM>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 8, SM>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Launch over the (d, nsplit) variants; sets the XCD mapping.  (D64: whether
// the d = 64 variants exist.)
template <int SM, bool D64 = true>
hipError_t prefill_bf16_dispatch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  a.xcd_map = (a.nsplit > 1 && (BH * a.nsplit) % (8 * a.nsplit) == 0) ? 1 : 0;
  if (d == 128) {
    switch (a.nsplit) {
      case 1: return launch_nt<128, 128, SM>(a, BH, stream);
      case 2: return launch_nt<128, 64, SM>(a, BH, stream);
      case 4: return launch_nt<128, 32, SM>(a, BH, stream);
    }
  } else if (d == 64) {
    if constexpr (D64) {
      switch (a.nsplit) {
        case 1: return launch_nt<64, 64, SM>(a, BH, stream);
        case 2: return launch_nt<64, 32, SM>(a, BH, stream);
      }
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace lal
