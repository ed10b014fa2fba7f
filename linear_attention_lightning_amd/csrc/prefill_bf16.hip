// Chunked ("Lightning") causal linear-attention prefill on bf16 matrix cores.
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
// Work decomposition.  One workgroup (8 waves) owns one (batch, head)
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
//  * Q rows are loaded by each wave straight into the registers that feed the
//    matrix cores, one block ahead (issued after the output phase, so that
//    they occupy registers only during the state update).
//  * LDS tiles are unpadded with an XOR swizzle of their 16-byte chunks,
//    chosen so that 16-byte fragment reads (one row per lane) and the
//    transposing 8-byte reads both run without bank conflicts.
//
// Products (all v_mfma_f32_16x16x32_bf16).  Outputs are computed transposed,
// O^T = S^T Q^T + V^T P^T, so a lane holds four consecutive value features of
// one token and stores 8 bytes.  P^T = K Q^T lands directly in the B-operand
// layout of V^T P^T.  K^T and V are read token-major with ds_read_b64_tr_b16.
//
// Balance.  Phase A (outputs) pairs row tiles t and NT-1-t so that every
// wave has the same causal work, and splits value columns across the waves
// of a pair; phase B (state update) spreads the state over a 4 x 2 grid of
// waves.  The number of 16-row tiles per block, NT, is a template parameter
// so that every loop bound is a compile-time constant.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlkMax = 128;

// Physical 16-byte chunk of logical chunk c in row r of a tile whose rows
// hold CPR chunks (an involution).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR == 16)
    return c ^ ((r & 7) << 1);
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
// the buffer land at LDS byte address lds_base + 16 l.  Issued from inline
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
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(desc), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) const char *)p);
}

// Wait until at most n vector-memory operations of this wave are in flight
// (they complete in issue order).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
  }
}

template <int D, int DV, int NT>
struct Plan {
  static constexpr int CPRK = D / 8;   // 16-byte chunks per K row / state-copy row
  static constexpr int CPRV = DV / 8;  // per V-slice row
  static constexpr int NJ = DV / 16;
  static constexpr int NI = D / 16;
  static constexpr int NKC = D / 32;
  static constexpr int BLKP = NT * 16;  // staged rows per block, a multiple of 32
  static constexpr int NCC = BLKP / 32;
  // phase A: RG row-tile pairs x CG column groups
  static constexpr int RG = NT / 2;
  static constexpr int CG0 = kWaves / RG;
  static constexpr int CG = CG0 < NJ ? CG0 : NJ;
  static constexpr int NJC = NJ / CG;
  static constexpr int AWAVES = RG * CG;
  // phase B: 4 x 2 grid of waves over the state tiles
  static constexpr int BIT = NI / 4;
  static constexpr int BJT = NJ / 2;
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
  static_assert(N_DMA <= 8, "vmcnt immediate");
  static_assert(NT % 2 == 0 && NT >= 2 && NT <= 8, "2..8 row tiles per block");
  static_assert(NJ % CG == 0 && AWAVES <= kWaves, "phase A grid");
  static_assert(BIT >= 1 && BJT >= 1, "phase B grid");
  static_assert(BLKP % KRPI == 0 && BLKP % VRPI == 0, "direct-load rows");
};

template <int D, int DV, int NT>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillArgs a) {
  using P = Plan<D, DV, NT>;
  // Two stages of K and V tiles, and the bf16 copy of the state slice.
  __shared__ __attribute__((aligned(1024))) u16 Ks0[kBlkMax * D];
  __shared__ __attribute__((aligned(1024))) u16 Ks1[kBlkMax * D];
  __shared__ __attribute__((aligned(1024))) u16 Vs0[kBlkMax * DV];
  __shared__ __attribute__((aligned(1024))) u16 Vs1[kBlkMax * DV];
  __shared__ __attribute__((aligned(1024))) u16 SsT[DV * D];  // SsT[j][i] = bf16(S[i][j0 + j])

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
  const int j0 = split * DV;
  const int64_t N = a.N;
  const int blk = a.blk;
  // Block bookkeeping in 32-bit scalars (the host guarantees N / blk < 2^31).
  const int nfull = (int)(N / blk);                       // blocks of blk tokens
  const int last = (int)(N - (int64_t)nfull * blk);       // tokens in a final partial block
  const int nblk = nfull + (last > 0 ? 1 : 0);

  const u16 *qh = a.q + (size_t)bh * (size_t)N * D;
  const u16 *kh = a.k + (size_t)bh * (size_t)N * D;
  const u16 *vh = a.v + (size_t)bh * (size_t)N * D;  // slice offset j0 added per load
  u16 *oh = a.o + (size_t)bh * (size_t)N * D + j0;
  float *Sh = a.state + (size_t)bh * D * D + j0;

  constexpr int RB = D * 2;    // bytes per K row and per state-copy row
  constexpr int VRB = DV * 2;  // bytes per V-slice row

  // ---- phase B ownership: i-tiles [ib*BIT, +BIT) x j-tiles [jb*BJT, +BJT) ----
  const int ib = wave & 3, jb = wave >> 2;
  f32x4 S_acc[P::BIT][P::BJT];
#pragma unroll
  for (int x = 0; x < P::BIT; ++x)
#pragma unroll
    for (int y = 0; y < P::BJT; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_acc[x][y][e] = Sh[(size_t)((ib * P::BIT + x) * 16 + 4 * g + e) * D + (jb * P::BJT + y) * 16 + lr];

  // ---- phase A role: row tiles {rg, NT-1-rg} x value tiles [jc0, jc0 + NJC) ----
  const bool act = wave < P::AWAVES;
  const int rg = wave % P::RG;
  const int jc0 = (wave / P::RG) * P::NJC;

  // ---- lane-constant LDS byte offsets ----
  // Every tile row used below is a multiple of 16 plus a lane-dependent part,
  // and the swizzle only looks at the low 4 row bits, so each access is a
  // per-lane constant plus a compile-time row offset (an immediate).
  const int h = (lr & 3) >> 1, lo8 = 8 * (lr & 1);
  const int rr = 4 * g + (lr >> 2);  // row of a transposing read within 16
  int kfrag[P::NKC];                 // 16-byte fragment of row lr, chunk 4kc+g
#pragma unroll
  for (int kc = 0; kc < P::NKC; ++kc) kfrag[kc] = lr * RB + (swz<P::CPRK>(lr, 4 * kc + g) << 4);
  int vtrA[P::NJC];  // V^T operand of value tile jc0+jl
#pragma unroll
  for (int jl = 0; jl < P::NJC; ++jl) vtrA[jl] = rr * VRB + (swz<P::CPRV>(rr, 2 * (jc0 + jl) + h) << 4) + lo8;
  int ktrB[P::BIT], vtrB[P::BJT];  // K^T and V operands of phase B
#pragma unroll
  for (int x = 0; x < P::BIT; ++x) ktrB[x] = rr * RB + (swz<P::CPRK>(rr, 2 * (ib * P::BIT + x) + h) << 4) + lo8;
#pragma unroll
  for (int y = 0; y < P::BJT; ++y) vtrB[y] = rr * VRB + (swz<P::CPRV>(rr, 2 * (jb * P::BJT + y) + h) << 4) + lo8;
  const int qlane = (lr * D + 8 * g) * 2;  // Q fragment of row lr

  auto ld128 = [](const u16 *base, int off) { return *(const bf16x8 *)((const char *)base + off); };
  auto ldtr = [](const u16 *base, int off0, int off1) {
    return join_tr(lds_read_tr((const u16 *)((const char *)base + off0)),
                   lds_read_tr((const u16 *)((const char *)base + off1)));
  };

  auto write_state_copy = [&]() {
#pragma unroll
    for (int x = 0; x < P::BIT; ++x)
#pragma unroll
      for (int y = 0; y < P::BJT; ++y) {
        const int off = ((jb * P::BJT + y) * 16 + lr) * RB + (swz<P::CPRK>(lr, 2 * (ib * P::BIT + x) + (g >> 1)) << 4) +
                        8 * (g & 1);
        lds_store_b64((const char *)SsT + off, pack_bf16x4(S_acc[x][y]));
      }
  };

  // ---- Q rows of the wave's two row tiles (registers) ----
  bf16x8 bq[2][P::NKC], qn[2][P::NKC];
  auto load_q = [&](auto rgi, int64_t tok0, int len) __attribute__((always_inline)) {
    constexpr int T[2] = {decltype(rgi)::value, NT - 1 - decltype(rgi)::value};
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh + (size_t)tok0 * D, len * D * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kc = 0; kc < P::NKC; ++kc)
        qn[u][kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rq, qlane, (16 * T[u] * D + kc * 32) * 2, 0));
  };

  // ---- direct HBM -> LDS loads of the K and V tiles of one block ----
  // Rows past len (a partial last block) and the padding slots read zeros.
  auto issue_kv = [&](int64_t tok0, int len, u16 *Kd, u16 *Vd) __attribute__((always_inline)) {
    const u32x4 dk = raw_desc(kh + (size_t)tok0 * D, (uint32_t)len * D * 2);
    const u32x4 dv = raw_desc(vh + (size_t)tok0 * D, (uint32_t)len * D * 2);
    const u32x4 none = raw_desc(kh, 0);
#pragma unroll
    for (int m = 0; m < P::KI_W; ++m) {
      const int inst = wave + kWaves * m;
      const int row = inst * P::KRPI + lane / P::CPRK;
      const int c = swz<P::CPRK>(row, lane % P::CPRK);
      dma_b128(inst < P::KINST ? dk : none, (row * D + c * 8) * 2, lds_addr(Kd + inst * 512));
    }
#pragma unroll
    for (int m = 0; m < P::VI_W; ++m) {
      const int inst = wave + kWaves * m;
      const int row = inst * P::VRPI + lane / P::CPRV;
      const int c = swz<P::CPRV>(row, lane % P::CPRV);
      dma_b128(inst < P::VINST ? dv : none, (row * D + j0 + c * 8) * 2, lds_addr(Vd + inst * 512));
    }
  };
  auto block_len = [&](int jb) { return jb < nfull ? blk : last; };


  // ---- phase A for row-tile pair {RGI, NT-1-RGI}: output rows ----
  auto phase_a = [&](auto rgi, int64_t tok0, int len, int nlen, const u16 *Kc, const u16 *Vc)
                     __attribute__((always_inline)) {
    constexpr int T[2] = {decltype(rgi)::value, NT - 1 - decltype(rgi)::value};
    f32x4 acc[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) acc[u][jl] = f32x4{0.f, 0.f, 0.f, 0.f};

    // inter-block part: O^T += S^T Q^T (each state operand feeds both row tiles)
#pragma unroll
    for (int kc = 0; kc < P::NKC; ++kc) {
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) {
        const bf16x8 as = ld128(SsT, kfrag[kc] + (jc0 + jl) * 16 * RB);
        acc[0][jl] = mfma_16x16x32(as, bq[0][kc], acc[0][jl]);
        acc[1][jl] = mfma_16x16x32(as, bq[1][kc], acc[1][jl]);
      }
    }

    // intra-block part, 32 keys at a time: O^T += V^T (P ⊙ M)^T.  Chunk cc
    // holds keys 32cc .. 32cc+31; row tile t uses chunks 0 .. t/2, and only
    // its last chunk straddles the diagonal.
#pragma unroll
    for (int cc = 0; cc <= T[1] / 2; ++cc) {
      const int c0 = 32 * cc;
      bf16x8 va[P::NJC];
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) va[jl] = ldtr(Vc, vtrA[jl] + c0 * VRB, vtrA[jl] + (c0 + 16) * VRB);
      // pt[u][s][e] = P[16 T_u + lr][c0 + 16 s + 4g + e]   (P^T = K Q^T)
      f32x4 pt[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bool need0 = cc <= T[0] / 2 && 2 * cc + s <= T[0];
        const bool need1 = 2 * cc + s <= T[1];
        if (!need0 && !need1) {
          pt[0][s] = pt[1][s] = f32x4{0.f, 0.f, 0.f, 0.f};
          continue;
        }
        bf16x8 ka[P::NKC];
#pragma unroll
        for (int kc = 0; kc < P::NKC; ++kc) ka[kc] = ld128(Kc, kfrag[kc] + (c0 + 16 * s) * RB);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          pt[u][s] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (u == 0 ? need0 : need1) {
#pragma unroll
            for (int kc = 0; kc < P::NKC; ++kc) pt[u][s] = mfma_16x16x32(ka[kc], bq[u][kc], pt[u][s]);
          }
        }
      }
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
        for (int jl = 0; jl < P::NJC; ++jl) acc[u][jl] = mfma_16x16x32(va[jl], pb, acc[u][jl]);
      }
    }

    uint2 packed[2][P::NJC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl) packed[u][jl] = pack_bf16x4(acc[u][jl]);

    // The next block's Q rows, issued only now so that their registers are not
    // live during the products above, and before this block's output stores,
    // so that waiting for them later leaves the stores' latency hidden.
    __builtin_amdgcn_sched_barrier(0);
    load_q(rgi, tok0 + blk, nlen);
    __builtin_amdgcn_sched_barrier(0);

    // store: acc[u][jl][e] = O[16 T_u + lr][(jc0 + jl) * 16 + 4g + e].  Rows
    // past len fall outside the descriptor and are dropped, so every wave
    // issues the same stores on every block.
    const u32x4 dod = raw_desc(oh + (size_t)tok0 * D, (uint32_t)(len * D - j0) * 2);
    __amdgpu_buffer_rsrc_t ro;
    __builtin_memcpy(&ro, &dod, sizeof(ro));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 16 * T[u] + lr;
#pragma unroll
      for (int jl = 0; jl < P::NJC; ++jl)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, packed[u][jl]), ro, ((r * D + (jc0 + jl) * 16 + 4 * g) * 2), 0, 0);
    }
  };

  // Call f(integral_constant<int, rg>) for the wave's row-tile pair.
  auto with_rg = [&](auto &&f) __attribute__((always_inline)) {
    if (rg == 0) f(std::integral_constant<int, 0>{});
    if constexpr (P::RG > 1) if (rg == 1) f(std::integral_constant<int, (P::RG > 1 ? 1 : 0)>{});
    if constexpr (P::RG > 2) if (rg == 2) f(std::integral_constant<int, (P::RG > 2 ? 2 : 0)>{});
    if constexpr (P::RG > 3) if (rg == 3) f(std::integral_constant<int, (P::RG > 3 ? 3 : 0)>{});
  };

  // ---- one block.  On entry the direct loads of block jblk (into Kc, Vc)
  // and, if it exists, of block jblk+1 (into the other stage) are in flight.
  // On exit the loads of block jblk+2 into (Kc, Vc) have been issued. ----
  auto body = [&](int jblk, const u16 *Kc, const u16 *Vc) __attribute__((always_inline)) {
    const int64_t tok0 = (int64_t)jblk * blk;
    const int len = block_len(jblk);
    // Everything issued before block jblk+1's direct loads (the last N_DMA
    // vector-memory operations of this wave, if that block exists) has
    // landed: this block's K/V tiles, its Q rows and the previous block's
    // output stores.
    if (jblk + 1 < nblk)
      wait_vmcnt(P::N_DMA);
    else
      wait_vmcnt(0);
    if (act) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kc = 0; kc < P::NKC; ++kc) bq[u][kc] = qn[u][kc];
    }
    lds_barrier();  // every wave's tiles of block jblk and the state copy are in LDS

    // ---------------- phase A: output rows (and the next block's Q) ----------------
    if (act) {
      const int nlen = jblk + 1 < nblk ? block_len(jblk + 1) : 0;
      with_rg([&](auto rgi) { phase_a(rgi, tok0, len, nlen, Kc, Vc); });
    }

    // ---------------- phase B: state update S += K^T V ----------------
#pragma unroll
    for (int cc = 0; cc < P::NCC; ++cc) {
      const int c0 = 32 * cc;
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

    // Every wave's reads of this stage and of the state copy are complete.
    // Only LDS accesses are drained: waiting for vector memory here would
    // also wait for block jblk+1's loads, which are still in flight.
    lds_barrier();
    write_state_copy();  // bf16 copy of S_jblk for the next block's phase A
    // Refill this stage with block jblk+2 while the LDS is otherwise idle.
    if (jblk + 2 < nblk) issue_kv(tok0 + 2 * (int64_t)blk, block_len(jblk + 2), (u16 *)Kc, (u16 *)Vc);
  };

  {
    const int len0 = block_len(0);
    if (act) with_rg([&](auto rgi) { load_q(rgi, 0, len0); });
    // The initial state is consumed here, before the loop, so the compiler's
    // waits for its loads stay out of the pipelined loop.
    write_state_copy();
    issue_kv(0, len0, Ks0, Vs0);
    if (nblk > 1) issue_kv(blk, block_len(1), Ks1, Vs1);
  }
  for (int jblk = 0; jblk < nblk; jblk += 2) {
    body(jblk, Ks0, Vs0);
    if (jblk + 1 < nblk) body(jblk + 1, Ks1, Vs1);
  }

  // ---- final state ----
#pragma unroll
  for (int x = 0; x < P::BIT; ++x)
#pragma unroll
    for (int y = 0; y < P::BJT; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Sh[(size_t)((ib * P::BIT + x) * 16 + 4 * g + e) * D + (jb * P::BJT + y) * 16 + lr] = S_acc[x][y][e];
}

template <int D, int DV>
hipError_t launch_nt(const PrefillArgs &a, int64_t BH, hipStream_t stream) {
  const int blkp = (a.blk + 31) & ~31;
  const dim3 grid((unsigned)(BH * a.nsplit)), block(kThreads);
  switch (blkp) {
    case 32: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 2>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 4>), grid, block, 0, stream, a); break;
    case 96: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 6>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int prefill_bf16_max_block(int) { return kBlkMax; }

int prefill_bf16_max_split(int d) { return d == 128 ? 4 : 2; }

hipError_t prefill_bf16_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  a.xcd_map = (a.nsplit > 1 && (BH * a.nsplit) % (8 * a.nsplit) == 0) ? 1 : 0;
  if (d == 128) {
    switch (a.nsplit) {
      case 1: return launch_nt<128, 128>(a, BH, stream);
      case 2: return launch_nt<128, 64>(a, BH, stream);
      case 4: return launch_nt<128, 32>(a, BH, stream);
    }
  } else if (d == 64) {
    switch (a.nsplit) {
      case 1: return launch_nt<64, 64>(a, BH, stream);
      case 2: return launch_nt<64, 32>(a, BH, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lal
