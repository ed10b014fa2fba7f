// Chunked causal linear-attention prefill with fp32 inputs and outputs.
//
// Same block decomposition as the bf16 kernel ("Почему M2 в итоге стала
// моделью с полным вниманием?" (ai.flicky.cc), section 1, glossary entry
// "Lightning Attention"; recurrence of "MiniMax-M1で理解する…" (zenn.dev),
// section "線形アテンションの数学的基礎"):
//
//   O_b = (Q_b K_b^T ⊙ M) V_b + Q_b S_{b-1},   S_b = S_{b-1} + K_b^T V_b,
//
// with every product and sum in fp32 on the vector ALUs, so that fp32 inputs
// keep fp32 accuracy.  One workgroup per sequence; the fp32 state, the K and
// V tiles of the current block, and 16-row slices of Q and P sit in LDS.
// This path serves small fp32 problems; it is not a throughput kernel.
//
// The gradient passes use it in other roles (as the bf16 kernel): the
// initial state from its own (optionally transposed) buffer, the final state
// to its own buffer or nowhere, and optionally the tokens in reversed order
// (logical token t is memory row N-1-t), where the causal mask becomes a
// suffix sum.
#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kThreads = 256;

template <int D>
struct CfgF32 {
  static constexpr int BLKMAX = (D == 128) ? 64 : 128;
  static constexpr int KSTR = D + 1;
  static constexpr int PSTR = BLKMAX + 1;
  static constexpr int S_OFF = 0;
  static constexpr int K_OFF = S_OFF + D * D;
  static constexpr int V_OFF = K_OFF + BLKMAX * KSTR;
  static constexpr int Q_OFF = V_OFF + BLKMAX * D;
  static constexpr int P_OFF = Q_OFF + 16 * KSTR;
  static constexpr int LDS_FLOATS = P_OFF + 16 * PSTR;
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_f32_kernel(PrefillF32Args a) {
  using C = CfgF32<D>;
  __shared__ float lds[C::LDS_FLOATS];
  float *Ss = lds + C::S_OFF;  // Ss[i][j]
  float *Ks = lds + C::K_OFF;  // Ks[c][i]
  float *Vs = lds + C::V_OFF;  // Vs[c][j]
  float *Qs = lds + C::Q_OFF;  // Qs[r][i], 16 rows
  float *Ps = lds + C::P_OFF;  // Ps[r][c], 16 rows

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t N = a.N;
  const int blk = a.blk;
  const float *qh = a.q + (size_t)bh * (size_t)N * D;
  const float *kh = a.k + (size_t)bh * (size_t)N * D;
  const float *vh = a.v + (size_t)bh * (size_t)N * D;
  float *oh = a.o + (size_t)bh * (size_t)N * D;
  float *Sh = a.grad ? nullptr : a.state + (size_t)bh * D * D;
  // memory row of logical token t
  auto mrow = [&](int64_t t) -> size_t { return (size_t)(a.rev ? N - 1 - t : t); };

  if (a.grad) {
    const float *gi = a.g_in ? a.g_in + (size_t)bh * D * D : nullptr;
    for (int idx = tid; idx < D * D; idx += kThreads)
      Ss[idx] = !gi ? 0.f : a.g_in_t ? gi[(idx % D) * D + idx / D] : gi[idx];
  } else {
    for (int idx = tid; idx < D * D; idx += kThreads) Ss[idx] = Sh[idx];
  }
  const int64_t nsnap = (a.snap && !a.grad) ? (N / blk) / a.snap_every : 0;

  for (int64_t tok0 = 0; tok0 < N; tok0 += blk) {
    const int len = (int)((N - tok0) < blk ? (N - tok0) : blk);
    __syncthreads();  // previous block's readers of Ks/Vs are done
    for (int idx = tid; idx < blk * D; idx += kThreads) {
      const int c = idx / D, i = idx % D;
      const bool ok = c < len;
      Ks[c * C::KSTR + i] = ok ? kh[mrow(tok0 + c) * D + i] : 0.f;
      Vs[c * D + i] = ok ? vh[mrow(tok0 + c) * D + i] : 0.f;
    }
    for (int rs = 0; rs < len; rs += 16) {
      __syncthreads();  // Ks/Vs staged; previous slice's readers of Qs/Ps done
      for (int idx = tid; idx < 16 * D; idx += kThreads) {
        const int r = idx / D, i = idx % D;
        Qs[r * C::KSTR + i] = (rs + r < len) ? qh[mrow(tok0 + rs + r) * D + i] : 0.f;
      }
      __syncthreads();
      // P[r][c] = q_r . k_c for c <= rs + r (inclusive causal mask), else 0
      for (int idx = tid; idx < 16 * blk; idx += kThreads) {
        const int r = idx / blk, c = idx % blk;
        float p = 0.f;
        if (c <= rs + r) {
          for (int i = 0; i < D; ++i) p = fmaf(Qs[r * C::KSTR + i], Ks[c * C::KSTR + i], p);
        }
        Ps[r * C::PSTR + c] = p;
      }
      __syncthreads();
      // O[r][j] = sum_c P[r][c] V[c][j] + sum_i Q[r][i] S[i][j]
      for (int idx = tid; idx < 16 * D; idx += kThreads) {
        const int r = idx / D, j = idx % D;
        if (rs + r >= len) continue;
        float intra = 0.f, inter = 0.f;
        for (int c = 0; c <= rs + r; ++c) intra = fmaf(Ps[r * C::PSTR + c], Vs[c * D + j], intra);
        for (int i = 0; i < D; ++i) inter = fmaf(Qs[r * C::KSTR + i], Ss[i * D + j], inter);
        oh[mrow(tok0 + rs + r) * D + j] = intra + inter;
      }
    }
    __syncthreads();  // every reader of the old state is done
    // S[i][j] += sum_c K[c][i] V[c][j]
    for (int idx = tid; idx < D * D; idx += kThreads) {
      const int i = idx / D, j = idx % D;
      float s = 0.f;
      for (int c = 0; c < len; ++c) s = fmaf(Ks[c * C::KSTR + i], Vs[c * D + j], s);
      Ss[idx] += s;
    }
    // snapshot of the state after this block (each thread copies the entries
    // it has just updated)
    const int64_t nb = tok0 / blk + 1;
    if (nsnap > 0 && nb % a.snap_every == 0 && nb / a.snap_every <= nsnap) {
      float *sp = a.snap + ((size_t)bh * nsnap + (nb / a.snap_every - 1)) * D * D;
      for (int idx = tid; idx < D * D; idx += kThreads) sp[idx] = Ss[idx];
    }
  }
  __syncthreads();
  if (a.grad) {
    if (a.g_out)
      for (int idx = tid; idx < D * D; idx += kThreads) a.g_out[(size_t)bh * D * D + idx] = Ss[idx];
  } else {
    for (int idx = tid; idx < D * D; idx += kThreads) Sh[idx] = Ss[idx];
  }
}

}  // namespace

int prefill_f32_max_block(int d) { return d == 128 ? CfgF32<128>::BLKMAX : CfgF32<64>::BLKMAX; }

hipError_t prefill_f32_launch(PrefillF32Args a, int64_t BH, int d, hipStream_t stream) {
  if (d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)BH), dim3(kThreads), 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)BH), dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lal
