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
// of its sequence in order.  The fp32 state slice S[:, j0:j0+DV] lives in
// matrix-core accumulators for the whole sequence (each wave owns some 16x16
// tiles of it) and is copied to LDS as bf16 once per block, as the operand of
// Q_b S.  Value-column slices of one sequence are independent except that
// each recomputes Q_b K_b^T; they exist to fill the GPU when B*H is small.
//
// All four products use v_mfma_f32_16x16x32_bf16.  Outputs are computed
// transposed (O^T = S^T Q^T + V^T P^T) so that a lane holds four consecutive
// value features of one token and stores 8 bytes.  The intra-block matrix is
// produced transposed, P^T = K Q^T, which lands directly in the B-operand
// layout of V^T P^T, so it never goes through LDS.  K^T and V are needed with
// tokens along the contraction; they are read from row-major LDS tiles with
// the transposing ds_read_b64_tr_b16.
//
// Staging.  Q, K and the V slice of block b+1 are loaded from HBM into
// registers while block b is computed, and written to LDS between the two
// barriers that separate blocks.  Rows past the end of the sequence and past
// the block are zero-filled, which makes ragged tails and block sizes that
// are not multiples of 32 exact without any other masking.
#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

template <int D, int DV>
struct Cfg {
  static constexpr int BLKMAX = (D == 128) ? 128 : 256;
  static constexpr int QSTR = D + 8;   // LDS row stride (elements) of Q, K tiles
  static constexpr int VSTR = DV + 8;  // of the V slice
  static constexpr int SSTR = D + 8;   // of the transposed bf16 state copy
  static constexpr int NJ = DV / 16;   // 16-wide value-column tiles
  static constexpr int NI = D / 16;    // 16-wide key-feature tiles
  static constexpr int NKC = D / 32;   // 32-wide chunks of the key features
  static constexpr int WPI = kWaves / NI;  // waves sharing one key-feature tile
  static constexpr int SJ = NJ / WPI;      // state column tiles per wave
  static constexpr int QCH = D / 8;        // 16-byte chunks per Q/K row
  static constexpr int VCH = DV / 8;       // per V-slice row
  static constexpr int PFQ = BLKMAX * QCH / kThreads;  // staged chunks per thread
  static constexpr int PFV = BLKMAX * VCH / kThreads;
  static constexpr int Q_OFF = 0;
  static constexpr int K_OFF = Q_OFF + BLKMAX * QSTR;
  static constexpr int V_OFF = K_OFF + BLKMAX * QSTR;
  static constexpr int S_OFF = V_OFF + BLKMAX * VSTR;
  static constexpr int LDS_ELEMS = S_OFF + DV * SSTR;
  static_assert(NI * WPI == kWaves, "key-feature tiles must split evenly over the waves");
  static_assert(SJ >= 1 && SJ * WPI == NJ, "state column tiles must split evenly");
  static_assert(PFQ * kThreads == BLKMAX * QCH && PFV * kThreads == BLKMAX * VCH, "staging split");
  static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS budget");
};

template <int D, int DV>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillArgs a) {
  using C = Cfg<D, DV>;
  __shared__ __attribute__((aligned(16))) u16 lds[C::LDS_ELEMS];
  u16 *Qs = lds + C::Q_OFF;
  u16 *Ks = lds + C::K_OFF;
  u16 *Vs = lds + C::V_OFF;
  u16 *SsT = lds + C::S_OFF;  // SsT[j][i] = bf16(S[i][j0 + j])

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (sequence, value slice).  With several slices per sequence
  // and a grid that is a multiple of 8 * nsplit, the slices of one sequence
  // get workgroup ids that are congruent mod 8, i.e. land on the same XCD
  // (workgroups are dispatched round-robin over the 8 XCDs), so their common
  // Q and K reads can hit that XCD's L2.
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
  const int blkp = (blk + 31) & ~31;  // LDS rows in use, a multiple of 32
  const int nt = blkp / 16;           // 16-row tiles per block
  const int64_t nblk = (N + blk - 1) / blk;

  const u16 *qh = a.q + (size_t)bh * (size_t)N * D;
  const u16 *kh = a.k + (size_t)bh * (size_t)N * D;
  const u16 *vh = a.v + (size_t)bh * (size_t)N * D + j0;
  u16 *oh = a.o + (size_t)bh * (size_t)N * D + j0;
  float *Sh = a.state + (size_t)bh * D * D + j0;

  // ---- state: load the fp32 slice owned by this wave into accumulators ----
  const int it = wave % C::NI;              // key-feature tile of this wave
  const int jb = (wave / C::NI) * C::SJ;    // first state column tile
  f32x4 S_acc[C::SJ];
#pragma unroll
  for (int s = 0; s < C::SJ; ++s) {
    const int jt = jb + s;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S_acc[s][e] = Sh[(size_t)(it * 16 + 4 * g + e) * D + jt * 16 + lr];
  }
  auto write_state_copy = [&]() {
#pragma unroll
    for (int s = 0; s < C::SJ; ++s) {
      const int jt = jb + s;
      *(uint2 *)&SsT[(jt * 16 + lr) * C::SSTR + it * 16 + 4 * g] = pack_bf16x4(S_acc[s]);
    }
  };
  write_state_copy();

  // ---- register staging of one block ----
  // Raw buffer loads through a descriptor that covers exactly the `len` valid
  // rows of the block: rows past the sequence end read as zero, with no
  // branches, so the loads stay in flight while the current block computes.
  u32x4 pq[C::PFQ], pk[C::PFQ], pv[C::PFV];
  auto load_block = [&](int64_t tok0, int len) {
    const int qk_bytes = len * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh + (size_t)tok0 * D, qk_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (size_t)tok0 * D, qk_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (size_t)tok0 * D, qk_bytes);
#pragma unroll
    for (int s = 0; s < C::PFQ; ++s) {
      const int id = tid + s * kThreads;
      const int off = ((id / C::QCH) * D + (id % C::QCH) * 8) * 2;
      pq[s] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      pk[s] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < C::PFV; ++s) {
      const int id = tid + s * kThreads;
      const int off = ((id / C::VCH) * D + (id % C::VCH) * 8) * 2;
      pv[s] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  };
  // All BLKMAX rows are written; rows past the block read as zero above.
  auto store_block = [&]() {
#pragma unroll
    for (int s = 0; s < C::PFQ; ++s) {
      const int id = tid + s * kThreads;
      const int row = id / C::QCH, ch = id % C::QCH;
      *(u32x4 *)&Qs[row * C::QSTR + ch * 8] = pq[s];
      *(u32x4 *)&Ks[row * C::QSTR + ch * 8] = pk[s];
    }
#pragma unroll
    for (int s = 0; s < C::PFV; ++s) {
      const int id = tid + s * kThreads;
      const int row = id / C::VCH, ch = id % C::VCH;
      *(u32x4 *)&Vs[row * C::VSTR + ch * 8] = pv[s];
    }
  };

  {
    const int len0 = (int)(N < blk ? N : blk);
    load_block(0, len0);
    store_block();
  }
  __syncthreads();

  // Row tiles of phase A: within each group of 8 tiles, tiles s and 7-s go to
  // the two waves that share SIMD s (waves w and w+4), balancing the causal
  // work per SIMD.
  const int t_first = (wave < 4) ? wave : 11 - wave;

  for (int64_t jblk = 0; jblk < nblk; ++jblk) {
    const int64_t tok0 = jblk * blk;
    const int len = (int)((N - tok0) < blk ? (N - tok0) : blk);
    const bool has_next = jblk + 1 < nblk;
    if (has_next) {
      const int64_t nt0 = tok0 + blk;
      load_block(nt0, (int)((N - nt0) < blk ? (N - nt0) : blk));
    }

    // ---------------- phase A: output rows ----------------
    for (int t = t_first; t < nt; t += 8) {
      const int r0 = t * 16;
      const int r = r0 + lr;  // this lane's token within the block
      bf16x8 bq[C::NKC];
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc)
        bq[kc] = *(const bf16x8 *)&Qs[r * C::QSTR + kc * 32 + 8 * g];
      f32x4 acc[C::NJ];
#pragma unroll
      for (int jt = 0; jt < C::NJ; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // inter-block part: O^T += S^T Q^T.  The scheduling barriers bound how
      // many operand loads the compiler hoists, keeping the prefetched next
      // block in registers instead of scratch.
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
#pragma unroll
        for (int jt = 0; jt < C::NJ; ++jt) {
          const bf16x8 as = *(const bf16x8 *)&SsT[(jt * 16 + lr) * C::SSTR + kc * 32 + 8 * g];
          acc[jt] = mfma_16x16x32(as, bq[kc], acc[jt]);
          if ((jt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      // intra-block part: O^T += V^T (P ⊙ M)^T, 32 key tokens at a time
      const int ncc = t / 2 + 1;
      for (int cc = 0; cc < ncc; ++cc) {
        const int c0 = cc * 32;
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < C::NKC; ++kc) {
          const bf16x8 ak = *(const bf16x8 *)&Ks[(c0 + lr) * C::QSTR + kc * 32 + 8 * g];
          p0 = mfma_16x16x32(ak, bq[kc], p0);
        }
        if (2 * cc + 1 <= t) {
#pragma unroll
          for (int kc = 0; kc < C::NKC; ++kc) {
            const bf16x8 ak = *(const bf16x8 *)&Ks[(c0 + 16 + lr) * C::QSTR + kc * 32 + 8 * g];
            p1 = mfma_16x16x32(ak, bq[kc], p1);
          }
        }
        // p0[e] = P[r][c0 + 4g + e], p1[e] = P[r][c0 + 16 + 4g + e]; keep c <= r
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[e] = (c0 + 4 * g + e <= r) ? (bf16)p0[e] : (bf16)0.f;
          pb[4 + e] = (c0 + 16 + 4 * g + e <= r) ? (bf16)p1[e] : (bf16)0.f;
        }
        // V^T operand with the same token order: slots 0..3 = rows c0+4g+e,
        // slots 4..7 = rows c0+16+4g+e, column jt*16 + lr.
        const int vrow = c0 + 4 * g + (lr >> 2);
        const int vcol = 4 * (lr & 3);
#pragma unroll
        for (int jt = 0; jt < C::NJ; ++jt) {
          const s16x4 lo = lds_read_tr(&Vs[vrow * C::VSTR + jt * 16 + vcol]);
          const s16x4 hi = lds_read_tr(&Vs[(vrow + 16) * C::VSTR + jt * 16 + vcol]);
          acc[jt] = mfma_16x16x32(join_tr(lo, hi), pb, acc[jt]);
          if ((jt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      // store: acc[jt][e] = O[r][jt*16 + 4g + e]
      if (r < len) {
        u16 *orow = oh + (size_t)(tok0 + r) * D;
#pragma unroll
        for (int jt = 0; jt < C::NJ; ++jt) *(uint2 *)(orow + jt * 16 + 4 * g) = pack_bf16x4(acc[jt]);
      }
    }

    // ---------------- phase B: state update S += K^T V ----------------
    {
      const int krow = 8 * g + (lr >> 2);
      const int col4 = 4 * (lr & 3);
      for (int c0 = 0; c0 < blkp; c0 += 32) {
        const s16x4 klo = lds_read_tr(&Ks[(c0 + krow) * C::QSTR + it * 16 + col4]);
        const s16x4 khi = lds_read_tr(&Ks[(c0 + krow + 4) * C::QSTR + it * 16 + col4]);
        const bf16x8 ak = join_tr(klo, khi);
#pragma unroll
        for (int s = 0; s < C::SJ; ++s) {
          const int jt = jb + s;
          const s16x4 vlo = lds_read_tr(&Vs[(c0 + krow) * C::VSTR + jt * 16 + col4]);
          const s16x4 vhi = lds_read_tr(&Vs[(c0 + krow + 4) * C::VSTR + jt * 16 + col4]);
          S_acc[s] = mfma_16x16x32(ak, join_tr(vlo, vhi), S_acc[s]);
        }
      }
    }

    __syncthreads();  // every read of this block's tiles and state copy is done
    write_state_copy();
    if (has_next) store_block();
    __syncthreads();
  }

  // ---- final state ----
#pragma unroll
  for (int s = 0; s < C::SJ; ++s) {
    const int jt = jb + s;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Sh[(size_t)(it * 16 + 4 * g + e) * D + jt * 16 + lr] = S_acc[s][e];
  }
}

template <int D, int DV>
hipError_t launch(const PrefillArgs &a, int64_t BH, hipStream_t stream) {
  const int64_t grid = BH * a.nsplit;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, DV>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int prefill_bf16_max_block(int d) { return d == 128 ? Cfg<128, 128>::BLKMAX : Cfg<64, 64>::BLKMAX; }

int prefill_bf16_max_split(int d) { return d == 128 ? 4 : 2; }

hipError_t prefill_bf16_launch(PrefillArgs a, int64_t BH, int d, hipStream_t stream) {
  a.xcd_map = (a.nsplit > 1 && (BH * a.nsplit) % (8 * a.nsplit) == 0) ? 1 : 0;
  if (d == 128) {
    switch (a.nsplit) {
      case 1: return launch<128, 128>(a, BH, stream);
      case 2: return launch<128, 64>(a, BH, stream);
      case 4: return launch<128, 32>(a, BH, stream);
    }
  } else if (d == 64) {
    switch (a.nsplit) {
      case 1: return launch<64, 64>(a, BH, stream);
      case 2: return launch<64, 32>(a, BH, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lal
