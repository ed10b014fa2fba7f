// Token-by-token causal linear-attention prefill with the state on chip.
//
// The recurrence S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t of
// "MiniMax-M1で理解する…" (zenn.dev/liushuzhi), section
// "線形アテンションの数学的基礎", applied one token at a time: 4 d^2 flop per
// token on the vector ALUs, no matrix cores.  It is the sequential baseline
// that the tiled kernel is measured against.
//
// Value columns of the state are independent, so a workgroup owns one
// (sequence, COLS-column slice): each of its 256 threads keeps COLS * d / 256
// fp32 state entries of one column in registers.  16-column slices are used
// when they give every compute unit a workgroup; fewer sequences get 8-column
// slices and twice the workgroups (8 heads of d = 128: 128 instead of 64).
// Each workgroup stages whole q and k rows, so narrower slices cost more
// staging and are slower once the GPU is full.  Tokens are processed in batches of 32:
// q, k and the v slice of a batch are staged in LDS, each thread runs the
// recurrence over the batch and leaves its partial o_t (a sum over its rows)
// in LDS, and the partials are then reduced and stored.  The next batch's q,
// k and v are loaded (16-byte pieces) into registers while a batch is
// computed, so only the first batch waits for memory.
#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 32;      // tokens per batch

template <int D, bool IO_BF16, int COLS>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(RecurrentArgs a) {
  constexpr int kCols = COLS;                 // value columns per workgroup
  constexpr int kGroups = kThreads / kCols;   // row groups (threads per column)
  constexpr int RPT = D / kGroups;            // state rows per thread
  __shared__ float2 qk[kTB][D];
  __shared__ float vv[kTB][kCols];
  __shared__ float red[kTB][kGroups][kCols + 1];

  const int tid = threadIdx.x;
  const int jj = tid % kCols;
  const int rg = tid / kCols;
  constexpr int nslice = D / kCols;
  const int64_t bh = blockIdx.x / nslice;
  const int j0 = (int)(blockIdx.x % nslice) * kCols;
  const int64_t N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  float *Sh = a.state + (size_t)bh * D * D;

  float S[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) S[m] = Sh[(size_t)(rg + kGroups * m) * D + j0 + jj];

  // a batch's q, k and v slice in 16-byte pieces of EPC elements: QP pieces of
  // q and of k per thread, and one v piece for the first VP threads.  Pieces
  // of tokens at or past N are zero.
  constexpr int EPC = IO_BF16 ? 8 : 4;
  constexpr int QP = kTB * D / EPC / kThreads;
  constexpr int VP = kTB * kCols / EPC;
  static_assert(QP * EPC * kThreads == kTB * D && VP <= kThreads && kCols % EPC == 0, "batch pieces");
  constexpr int ES = IO_BF16 ? 2 : 4;
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
      const int tt = tid * EPC / kCols, c0 = tid * EPC % kCols;
      if (tok0 + tt < N) vp = *(const u32x4 *)((const char *)a.v + (base + (size_t)(tok0 + tt) * D + j0 + c0) * ES);
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
      for (int e = 0; e < EPC; ++e) qk[tt][i0 + e] = make_float2(elem(qp[j], e), elem(kp[j], e));
    }
    if (tid < VP) {
      const int tt = tid * EPC / kCols, c0 = tid * EPC % kCols;
#pragma unroll
      for (int e = 0; e < EPC; ++e) vv[tt][c0 + e] = elem(vp, e);
    }
    __syncthreads();
    if (tok0 + kTB < N) load_batch(tok0 + kTB);  // in flight during this batch
    for (int tt = 0; tt < n; ++tt) {
      const float vj = vv[tt][jj];
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const float2 x = qk[tt][rg + kGroups * m];
        S[m] = fmaf(x.y, vj, S[m]);   // S_t = S_{t-1} + k_t v_t^T
        part = fmaf(x.x, S[m], part);  // partial of q_t^T S_t
      }
      red[tt][rg][jj] = part;
    }
    __syncthreads();
    for (int idx = tid; idx < n * kCols; idx += kThreads) {
      const int tt = idx / kCols, c = idx % kCols;
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < kGroups; ++r) o += red[tt][r][c];
      const size_t oi = base + (size_t)(tok0 + tt) * D + j0 + c;
      if constexpr (IO_BF16)
        ((u16 *)a.o)[oi] = f32_to_bf16_bits(o);
      else
        ((float *)a.o)[oi] = o;
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) Sh[(size_t)(rg + kGroups * m) * D + j0 + jj] = S[m];
}

// 16-column slices when they alone give every compute unit a workgroup,
// else 8-column slices (twice the workgroups)
template <int D, bool IO>
hipError_t go(const RecurrentArgs &a, int cus, hipStream_t stream) {
  if (a.BH * (D / 16) >= cus)
    hipLaunchKernelGGL((recurrent_kernel<D, IO, 16>), dim3((unsigned)(a.BH * (D / 16))), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<D, IO, 8>), dim3((unsigned)(a.BH * (D / 8))), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t recurrent_launch(RecurrentArgs a, int d, bool io_bf16, int cus, hipStream_t stream) {
  if (d == 128) return io_bf16 ? go<128, true>(a, cus, stream) : go<128, false>(a, cus, stream);
  if (d == 64) return io_bf16 ? go<64, true>(a, cus, stream) : go<64, false>(a, cus, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
