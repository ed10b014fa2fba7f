// Several decode tokens per sequence in two steps, for verifying T <= 16
// draft tokens (speculative decoding, the open problem that "ノーフリーランチ"
// (winzheng.jp), section "推論システム統合の課題", names for linear attention):
//
//  verify:  o_t = q_t^T S_t for t = 0 .. T-1, S_t = S + sum_{s <= t} k_s v_s^T,
//           computed as  q_t^T S  +  sum_{s <= t} (q_t . k_s) v_s  without
//           writing the state (the recurrence of "MiniMax-M1で理解する"
//           (zenn.dev/liushuzhi), section "線形アテンションの数学的基礎",
//           unrolled over the drafts);
//  commit:  S <- S + sum_{t < a} k_t v_t^T for the a drafts accepted by the
//           sequence (a = 0 leaves S as it was: the rollback).
//
// Both are a single streaming pass over the state (read; read and write), so
// verifying T drafts costs about one decode step of state traffic instead of
// T.  Layout as in the one-token decode: one wavefront per (batch, head),
// each lane owns 4 columns of the rows it walks (16-byte fp32 or 8-byte bf16
// state accesses); q and k of the drafts are staged in LDS (transposed, so a
// state row's T multipliers are contiguous).
//
// commit applies, per state element, the same fused multiply-adds in the
// same order as T one-token decode steps; with an fp32 state the result is
// bit-identical to them.  With a bf16 or OCP FP8 E4M3 state it rounds once,
// at the store.  Narrow states carry a per-sequence scale and are kept in
// stored units (state / scale) as in the one-token decode: verify multiplies
// the state part of its outputs by the scale, commit divides v by it.
#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kW = 4;       // wavefronts (sequences) per commit workgroup
constexpr int kWV = 2;      // per verify workgroup (its LDS staging is twice as large)
constexpr int kTMax = 16;   // drafts per call

template <bool BF16>
__device__ __forceinline__ float ld_io(const void *p, size_t i) {
  if constexpr (BF16)
    return bf16_bits_to_f32(((const u16 *)p)[i]);
  else
    return ((const float *)p)[i];
}

// 4 consecutive state entries as fp32
template <int ST>
__device__ __forceinline__ void ld_state4(const void *row, int cg, float (&s)[4]) {
  if constexpr (ST == kStE4M3) {
    const f32x4 w = e4m3x4_to_f32(__builtin_nontemporal_load((const uint32_t *)row + cg));
    s[0] = w[0];
    s[1] = w[1];
    s[2] = w[2];
    s[3] = w[3];
  } else if constexpr (ST == kStBF16) {
    const u32x2 w = __builtin_nontemporal_load((const u32x2 *)row + cg);
    s[0] = __uint_as_float(w[0] << 16);
    s[1] = __uint_as_float(w[0] & 0xffff0000u);
    s[2] = __uint_as_float(w[1] << 16);
    s[3] = __uint_as_float(w[1] & 0xffff0000u);
  } else {
    const f32x4 w = __builtin_nontemporal_load((const f32x4 *)row + cg);
    s[0] = w[0];
    s[1] = w[1];
    s[2] = w[2];
    s[3] = w[3];
  }
}

template <int ST>
__device__ __forceinline__ void st_state4(void *row, int cg, const float (&s)[4]) {
  if constexpr (ST == kStE4M3) {
    __builtin_nontemporal_store(f32_to_e4m3x4(f32x4{s[0], s[1], s[2], s[3]}), (uint32_t *)row + cg);
  } else if constexpr (ST == kStBF16) {
    const bf16x2 lo = {(bf16)s[0], (bf16)s[1]}, hi = {(bf16)s[2], (bf16)s[3]};
    const u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    __builtin_nontemporal_store(w, (u32x2 *)row + cg);
  } else {
    const f32x4 w = {s[0], s[1], s[2], s[3]};
    __builtin_nontemporal_store(w, (f32x4 *)row + cg);
  }
}

template <int D, bool IO_BF16, int ST>
__global__ __launch_bounds__(64 * kWV) void verify_kernel(DecodeMultiArgs a) {
  constexpr int ES = ST == kStF32 ? 4 : ST == kStBF16 ? 2 : 1;
  constexpr int LPR = D / 4;    // lanes per state row (4 columns each)
  constexpr int RP = 64 / LPR;  // rows per wave access
  constexpr int RPL = D / RP;   // rows per lane
  constexpr int U = 8;          // rows in flight per lane
  static_assert(RPL % U == 0, "row unroll");
  extern __shared__ float lds[];
  const int T = a.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float *qT = lds + (size_t)wave * (2 * D * T + kTMax * kTMax);  // qT[i * T + t]
  float *kT = qT + D * T;                                       // kT[i * T + s]
  float *P = kT + D * T;                                        // P[t * kTMax + s]
  const int64_t h = (int64_t)blockIdx.x * kWV + wave;
  const bool valid = h < a.BH;
  if (valid) {
    for (int x = lane; x < D * T; x += 64) {
      const int t = x / D, i = x % D;
      qT[i * T + t] = ld_io<IO_BF16>(a.q, ((size_t)h * T + t) * D + i);
      kT[i * T + t] = ld_io<IO_BF16>(a.k, ((size_t)h * T + t) * D + i);
    }
  }
  __syncthreads();
  if (!valid) return;

  // P[t][s] = q_t . k_s for s <= t
  for (int x = lane; x < T * T; x += 64) {
    const int t = x / T, s = x % T;
    float p = 0.f;
    if (s <= t)
      for (int i = 0; i < D; ++i) p = fmaf(qT[i * T + t], kT[i * T + s], p);
    P[t * kTMax + s] = p;
  }

  const int cg = lane % LPR, rph = lane / LPR;
  float acc[kTMax][4];
#pragma unroll
  for (int t = 0; t < kTMax; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[t][e] = 0.f;

  const char *Sh = (const char *)a.state + (size_t)h * D * D * ES;
  for (int m0 = 0; m0 < RPL; m0 += U) {
    float s[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) ld_state4<ST>(Sh + (size_t)(rph + RP * (m0 + u)) * D * ES, cg, s[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float *qi = qT + (rph + RP * (m0 + u)) * T;
#pragma unroll
      for (int t = 0; t < kTMax; ++t) {
        if (t < T) {
          const float qv = qi[t];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(qv, s[u][e], acc[t][e]);
        }
      }
    }
  }
  // lanes with equal cg hold partial sums over disjoint rows
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int t = 0; t < kTMax; ++t)
      if (t < T)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] += __shfl_xor(acc[t][e], off, 64);
  if constexpr (ST != kStF32) {
    // the state part was read in stored units
    const float sc = a.scale ? a.scale[h] : 1.f;
#pragma unroll
    for (int t = 0; t < kTMax; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] *= sc;
  }
  // P was written by other lanes of this wavefront: its LDS stores precede
  // the reads below in the wavefront's in-order LDS queue once drained
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  if (rph == 0) {
    // within the drafts: o_t += sum_{s <= t} P[t][s] v_s
#pragma unroll
    for (int s = 0; s < kTMax; ++s) {
      if (s < T) {
        float vs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vs[e] = ld_io<IO_BF16>(a.v, ((size_t)h * T + s) * D + 4 * cg + e);
#pragma unroll
        for (int t = 0; t < kTMax; ++t) {
          if (t >= s && t < T) {
            const float p = P[t * kTMax + s];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(p, vs[e], acc[t][e]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kTMax; ++t) {
      if (t < T) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t oi = ((size_t)h * T + t) * D + 4 * cg + e;
          if constexpr (IO_BF16)
            ((u16 *)a.o)[oi] = f32_to_bf16_bits(acc[t][e]);
          else
            ((float *)a.o)[oi] = acc[t][e];
        }
      }
    }
  }
}

template <int D, bool IO_BF16, int ST>
__global__ __launch_bounds__(64 * kW) void commit_kernel(DecodeMultiArgs a) {
  constexpr int ES = ST == kStF32 ? 4 : ST == kStBF16 ? 2 : 1;
  constexpr int LPR = D / 4;
  constexpr int RP = 64 / LPR;
  constexpr int RPL = D / RP;
  constexpr int U = 8;
  static_assert(RPL % U == 0, "row unroll");
  extern __shared__ float lds[];
  const int T = a.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float *kT = lds + (size_t)wave * D * T;  // kT[i * T + t]
  const int64_t h = (int64_t)blockIdx.x * kW + wave;
  const bool valid = h < a.BH;
  int cnt = 0;
  if (valid) {
    cnt = a.accept ? a.accept[h / a.H] : T;
    cnt = cnt < 0 ? 0 : (cnt > T ? T : cnt);
    for (int x = lane; x < D * T; x += 64) {
      const int t = x / D, i = x % D;
      kT[i * T + t] = ld_io<IO_BF16>(a.k, ((size_t)h * T + t) * D + i);
    }
  }
  __syncthreads();
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if (!valid || cnt == 0) return;

  const int cg = lane % LPR, rph = lane / LPR;
  // narrow states are updated in stored units: v / scale
  const float inv = (ST != kStF32 && a.scale) ? 1.f / a.scale[h] : 1.f;
  float vr[kTMax][4];
#pragma unroll
  for (int t = 0; t < kTMax; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vr[t][e] = t < cnt ? ld_io<IO_BF16>(a.v, ((size_t)h * T + t) * D + 4 * cg + e) * inv : 0.f;

  char *Sh = (char *)a.state + (size_t)h * D * D * ES;
  for (int m0 = 0; m0 < RPL; m0 += U) {
    float s[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) ld_state4<ST>(Sh + (size_t)(rph + RP * (m0 + u)) * D * ES, cg, s[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = rph + RP * (m0 + u);
      const float *ki = kT + i * T;
#pragma unroll
      for (int t = 0; t < kTMax; ++t) {
        if (t < cnt) {
          const float kv = ki[t];
#pragma unroll
          for (int e = 0; e < 4; ++e) s[u][e] = fmaf(kv, vr[t][e], s[u][e]);
        }
      }
      st_state4<ST>(Sh + (size_t)i * D * ES, cg, s[u]);
    }
  }
}

template <int D, bool IO, int ST>
hipError_t go(const DecodeMultiArgs &a, bool commit, hipStream_t stream) {
  if (commit) {
    const int64_t grid = (a.BH + kW - 1) / kW;
    const size_t lds = (size_t)kW * D * a.T * sizeof(float);  // <= 32 KiB
    hipLaunchKernelGGL((commit_kernel<D, IO, ST>), dim3((unsigned)grid), dim3(64 * kW), lds, stream, a);
  } else {
    const int64_t grid = (a.BH + kWV - 1) / kWV;
    const size_t lds = (size_t)kWV * (2 * D * a.T + kTMax * kTMax) * sizeof(float);  // <= 34 KiB
    hipLaunchKernelGGL((verify_kernel<D, IO, ST>), dim3((unsigned)grid), dim3(64 * kWV), lds, stream, a);
  }
  return hipGetLastError();
}

template <int D, bool IO>
hipError_t go_st(const DecodeMultiArgs &a, bool commit, int st, hipStream_t stream) {
  switch (st) {
    case kStF32: return go<D, IO, kStF32>(a, commit, stream);
    case kStBF16: return go<D, IO, kStBF16>(a, commit, stream);
    case kStE4M3: return go<D, IO, kStE4M3>(a, commit, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int decode_multi_max_tokens() { return kTMax; }

hipError_t decode_multi_launch(DecodeMultiArgs a, int d, bool commit, bool io_bf16, int state_fmt,
                               hipStream_t stream) {
  if (a.T < 1 || a.T > kTMax) return hipErrorInvalidValue;
  if (d == 128)
    return io_bf16 ? go_st<128, true>(a, commit, state_fmt, stream) : go_st<128, false>(a, commit, state_fmt, stream);
  if (d == 64)
    return io_bf16 ? go_st<64, true>(a, commit, state_fmt, stream) : go_st<64, false>(a, commit, state_fmt, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
