// Token-by-token causal linear-attention prefill with the state on chip.
//
// The recurrence S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t of
// "MiniMax-M1で理解する…" (zenn.dev/liushuzhi), section
// "線形アテンションの数学的基礎", applied one token at a time: 4 d^2 flop per
// token on the vector ALUs, no matrix cores.  It is the sequential baseline
// that the tiled kernel is measured against.
//
// Value columns of the state are independent, so a workgroup owns one
// (sequence, C-column slice).  Its 256 threads are 256 / C row groups times
// C columns; a thread keeps RPT = d C / 256 consecutive rows of one column in
// registers.  C is the widest of 16, 8 and 4 columns that still gives every
// compute unit a workgroup (8 heads of d = 128: 4 columns, 256 workgroups);
// wider slices stage each q and k row for more columns.
//
// Tokens are processed in batches of 32.  A batch's q and k are staged in
// LDS as (q_i, k_i) pairs, so that a thread's RPT rows are RPT pairs in a
// row (16-byte reads; the rows are padded against bank conflicts), and its v
// slice transposed beside them (a column's 32
// values in a row).  The batch loop is unrolled over all 32 tokens (tokens at
// or past N are zero, and change nothing), in groups whose reads are issued
// one group ahead of the arithmetic: the LDS latency is hidden with one wave
// per SIMD.  Each
// thread leaves its partial q_t^T S_t (a sum over its rows) in LDS; after
// the batch the partials are summed and the outputs stored.  The next
// batch's q, k and v are loaded (16-byte pieces) into registers while a
// batch is computed, so only the first batch waits for memory.
#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 32;  // tokens per batch

template <int D, bool IO_BF16, int C>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(RecurrentArgs a) {
  constexpr int kGroups = kThreads / C;  // row groups
  constexpr int RPT = D / kGroups;       // consecutive state rows per thread
  static_assert(RPT >= 1 && RPT <= 8 && RPT * kGroups == D, "rows per thread");
  // (q_i, k_i) pairs of a token's rows, 2 pairs (16 bytes) of padding after
  // every 8 rows: 8-row pieces then start 20 words apart, so 16 lanes storing
  // consecutive pieces hit 16 distinct bank positions
  constexpr int kQKRow = D + D / 4;  // float2 per token
  __shared__ __attribute__((aligned(16))) float2 qk[kTB * kQKRow];
  auto qk_at = [](int tt, int r) { return tt * kQKRow + r + (r >> 3) * 2; };
  // v transposed (a column's batch contiguous), rows padded to spread them over the banks
  constexpr int kVRow = kTB + 4;
  __shared__ __attribute__((aligned(16))) float vv[C][kVRow];
  // partials: token tt, row group r, column c at tt (kThreads + C) + r C + c.
  // A wave's stores of one token are 64 consecutive words, and its loads of
  // one row group for 64 (token, column) outputs fall in 64 distinct banks.
  constexpr int kRedTok = kThreads + C;
  __shared__ float red[kTB * kRedTok];

  const int tid = threadIdx.x;
  const int jj = tid % C;
  const int rg = tid / C;
  const int r0 = rg * RPT;
  constexpr int nslice = D / C;
  const int64_t bh = blockIdx.x / nslice;
  const int j0 = (int)(blockIdx.x % nslice) * C;
  const int64_t N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  float *Sh = a.state + (size_t)bh * D * D;

  float S[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) S[m] = Sh[(size_t)(r0 + m) * D + j0 + jj];

  // a batch's q, k and v slice: QP 16-byte pieces of EPC elements of q and of
  // k per thread, and one v piece of VE elements (8 or 16 bytes) for the first
  // VP threads.  Pieces of tokens at or past N are zero.
  constexpr int EPC = IO_BF16 ? 8 : 4;
  constexpr int QP = kTB * D / EPC / kThreads;
  constexpr int VE = C < EPC ? C : EPC;
  constexpr int VP = kTB * C / VE;
  constexpr int ES = IO_BF16 ? 2 : 4;
  static_assert(QP * EPC * kThreads == kTB * D && VP <= kThreads && C % VE == 0 && (VE * ES == 16 || VE * ES == 8),
                "batch pieces");
  u32x4 qp[QP], kp[QP], vp;
  auto load_batch = [&](int64_t tok0) {
#pragma unroll
    for (int j = 0; j < QP; ++j) {
      const int c = tid + kThreads * j, tt = c * EPC / D, i0 = c * EPC % D;
      qp[j] = kp[j] = u32x4{0u, 0u, 0u, 0u};
      if (tok0 + tt < N) {
        const size_t off = (base + (size_t)(tok0 + tt) * D + i0) * ES;
        qp[j] = *(const u32x4 *)((const char *)a.q + off);
        kp[j] = *(const u32x4 *)((const char *)a.k + off);
      }
    }
    vp = u32x4{0u, 0u, 0u, 0u};
    if (tid < VP) {
      const int tt = tid * VE / C, c0 = tid * VE % C;
      if (tok0 + tt < N) {
        const char *src = (const char *)a.v + (base + (size_t)(tok0 + tt) * D + j0 + c0) * ES;
        if constexpr (VE * ES == 16) {
          vp = *(const u32x4 *)src;
        } else {
          const uint2 t = *(const uint2 *)src;
          vp = u32x4{t.x, t.y, 0u, 0u};
        }
      }
    }
  };
  auto elem = [&](const u32x4 &p, int e) -> float {
    if constexpr (IO_BF16)
      return __uint_as_float(e & 1 ? p[e / 2] & 0xffff0000u : p[e / 2] << 16);
    else
      return __uint_as_float(p[e]);
  };

  load_batch(0);
  for (int64_t tok0 = 0; tok0 < N; tok0 += kTB) {
    const int n = (int)((N - tok0) < kTB ? (N - tok0) : kTB);
#pragma unroll
    for (int j = 0; j < QP; ++j) {
      const int c = tid + kThreads * j, tt = c * EPC / D, i0 = c * EPC % D;
#pragma unroll
      for (int e = 0; e < EPC; e += 2)  // two (q, k) pairs per 16-byte store
        *(float4 *)&qk[qk_at(tt, i0 + e)] =
            make_float4(elem(qp[j], e), elem(kp[j], e), elem(qp[j], e + 1), elem(kp[j], e + 1));
    }
    if (tid < VP) {
      const int tt = tid * VE / C, c0 = tid * VE % C;
#pragma unroll
      for (int e = 0; e < VE; ++e) vv[c0 + e][tt] = elem(vp, e);
    }
    __syncthreads();
    if (tok0 + kTB < N) load_batch(tok0 + kTB);  // in flight during this batch
    // The batch in groups of G tokens, G 2 RPT operands each (~32 registers):
    // group g+1's (q, k) reads are issued before group g's arithmetic.
    float vj[kTB];
#pragma unroll
    for (int t4 = 0; t4 < kTB; t4 += 4) *(float4 *)&vj[t4] = *(const float4 *)&vv[jj][t4];
    constexpr int G = RPT >= 16 ? 1 : 16 / RPT;
    static_assert(kTB % G == 0, "token groups");
    float x[2][G][2 * RPT];
    auto load_group = [&](int g, float (&xg)[G][2 * RPT]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int tt = g * G + u;
        if constexpr (RPT == 1) {
          const float2 p = qk[qk_at(tt, r0)];
          xg[u][0] = p.x;
          xg[u][1] = p.y;
        } else {
#pragma unroll
          for (int m = 0; m < RPT; m += 2) {  // a thread's rows lie in one 8-row piece (RPT <= 8)
            const float4 p = *(const float4 *)&qk[qk_at(tt, r0) + m];
            xg[u][2 * m] = p.x;
            xg[u][2 * m + 1] = p.y;
            xg[u][2 * m + 2] = p.z;
            xg[u][2 * m + 3] = p.w;
          }
        }
      }
    };
    load_group(0, x[0]);
#pragma unroll
    for (int g = 0; g < kTB / G; ++g) {
      if (g + 1 < kTB / G) load_group(g + 1, x[(g + 1) & 1]);
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int tt = g * G + u;
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
          S[m] = fmaf(x[g & 1][u][2 * m + 1], vj[tt], S[m]);  // S_t = S_{t-1} + k_t v_t^T
          part = fmaf(x[g & 1][u][2 * m], S[m], part);        // partial of q_t^T S_t
        }
        red[tt * kRedTok + tid] = part;  // rg C + jj = tid
      }
    }
    __syncthreads();
    // Outputs: kTB C sums of kGroups partials.  Every thread takes an output
    // and 1/SPL of its partials (4 independent running sums); the SPL = 2
    // shares of an output sit in adjacent lanes and are combined across them.
    constexpr int SPL = kThreads / (kTB * C) >= 2 ? 2 : 1;
    constexpr int OPT2 = kTB * C * SPL / kThreads;  // outputs per thread
    constexpr int PR = kGroups / SPL;               // partials per share
    static_assert(OPT2 * kThreads == kTB * C * SPL && PR % 4 == 0, "output shares");
#pragma unroll
    for (int u = 0; u < OPT2; ++u) {
      const int idx = (tid + kThreads * u) / SPL, sh = tid % SPL;
      const int tt = idx / C, c = idx % C;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      const float *rp = &red[tt * kRedTok + sh * PR * C + c];
#pragma unroll
      for (int r = 0; r < PR; ++r) acc[r % 4] += rp[r * C];
      float o = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      if constexpr (SPL >= 2)  // the neighbour lane's share (DPP quad_perm [1,0,3,2])
        o += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(o), 0xb1, 0xf, 0xf, false));
      if (sh == 0 && tt < n) {
        const size_t oi = base + (size_t)(tok0 + tt) * D + j0 + c;
        if constexpr (IO_BF16)
          ((u16 *)a.o)[oi] = f32_to_bf16_bits(o);
        else
          ((float *)a.o)[oi] = o;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) Sh[(size_t)(r0 + m) * D + j0 + jj] = S[m];
}

template <int D, bool IO, int C>
hipError_t launch(const RecurrentArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((recurrent_kernel<D, IO, C>), dim3((unsigned)(a.BH * (D / C))), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// the widest slice that still gives every compute unit a workgroup
template <int D, bool IO>
hipError_t go(const RecurrentArgs &a, int cus, hipStream_t stream) {
  if (a.BH * (D / 16) >= cus) return launch<D, IO, 16>(a, stream);
  if (a.BH * (D / 8) >= cus) return launch<D, IO, 8>(a, stream);
  return launch<D, IO, 4>(a, stream);
}

}  // namespace

hipError_t recurrent_launch(RecurrentArgs a, int d, bool io_bf16, int cus, hipStream_t stream) {
  if (d == 128) return io_bf16 ? go<128, true>(a, cus, stream) : go<128, false>(a, cus, stream);
  if (d == 64) return io_bf16 ? go<64, true>(a, cus, stream) : go<64, false>(a, cus, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
