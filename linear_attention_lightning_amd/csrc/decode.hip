// One decode token per sequence: S <- S + k v^T, o = q^T S.
//
// The recurrence of "MiniMax-M1で理解する…" (zenn.dev/liushuzhi), section
// "線形アテンションの数学的基礎", with N = 1.  Section 4 of "Почему M2 в итоге
// стала моделью с полным вниманием?" (ai.flicky.cc) characterises this step:
// a small state matrix read and written every token while the GPU waits on
// memory.  It moves 2 d^2 state elements per 4 d^2 flop, so the kernel is a
// streaming read-modify-write of the state at HBM speed:
//
//  * one wavefront per (batch, head); four per 256-thread workgroup;
//  * each lane owns 16 bytes of a state row (4 fp32, 8 bf16 or 16 fp8
//    columns) and walks the rows that map to it, so every state access is a
//    coalesced, non-temporal 16-byte load or store;
//  * q_i and k_i are broadcast from LDS, v_j stays in registers;
//  * o_j accumulates per lane over its rows and is finished with a
//    cross-lane butterfly reduction.
//
// Narrow state storage (bf16, or OCP FP8 E4M3) with a per-sequence scale:
// each element is widened to fp32, updated with one fused multiply-add, read
// into o from the fp32 value, and stored back rounded to nearest even -- the
// low-precision state storage whose rounding drift "ノーフリーランチ：MiniMax
// M2が高効率アテンション機構を解体" (winzheng.jp), section "推論システム統合
// の課題", warns about.  The kernel keeps the state in stored units x / scale:
// v is divided and q multiplied by the scale once per sequence, so the
// per-element work is the same as without a scale (and exact for powers of
// two).
#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kWavesPerBlock = 4;

template <bool BF16>
__device__ __forceinline__ float load_io(const void *p, size_t i) {
  if constexpr (BF16)
    return bf16_bits_to_f32(((const u16 *)p)[i]);
  else
    return ((const float *)p)[i];
}

template <int D, bool IO_BF16, int ST>
__global__ __launch_bounds__(64 * kWavesPerBlock) void decode_kernel(DecodeArgs a) {
  constexpr int ES = ST == kStF32 ? 4 : ST == kStBF16 ? 2 : 1;  // bytes per state element
  constexpr int VE = 16 / ES;          // state elements per 16-byte access
  constexpr int LPR = D / VE;          // lanes covering one state row
  constexpr int RP = 64 / LPR;         // rows covered by one wave access
  constexpr int RPL = D / RP;          // rows per lane
  constexpr int U = RPL < 8 ? RPL : 8; // rows in flight per lane
  static_assert(RPL % U == 0, "row unroll");

  __shared__ float2 qk[kWavesPerBlock][D];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t h = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const bool valid = h < a.BH;
  // stored units: S' = S / scale (fp32 states are never scaled)
  const float sc = (ST != kStF32 && valid && a.scale) ? a.scale[h] : 1.f;
  const float inv = 1.f / sc;

  if (valid) {
    for (int i = lane; i < D; i += 64)
      qk[wave][i] = make_float2(load_io<IO_BF16>(a.q, (size_t)h * D + i) * sc,
                                load_io<IO_BF16>(a.k, (size_t)h * D + i));
  }
  __syncthreads();
  if (!valid) return;

  const int cg = lane % LPR;  // column group: columns cg*VE .. cg*VE+VE-1
  const int rph = lane / LPR; // rows rph, rph+RP, ...
  float vj[VE], acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    vj[e] = load_io<IO_BF16>(a.v, (size_t)h * D + cg * VE + e) * inv;
    acc[e] = 0.f;
  }

  u32x4 *Sh = (u32x4 *)((char *)a.state + (size_t)h * D * D * ES);  // 16-byte units
  constexpr int U16_PER_ROW = D * ES / 16;

  if constexpr (ST == kStE4M3) {
    // one batch of U rows per lane, the loop kept rolled: this form measured
    // 5 % faster than the loop over both batches written out
    auto rows = [&](int m0) {
      u32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = rph + RP * (m0 + u);
        raw[u] = __builtin_nontemporal_load(Sh + (size_t)i * U16_PER_ROW + cg);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = rph + RP * (m0 + u);
        const float2 qki = qk[wave][i];
        u32x4 w;
        // each 32-bit word holds four fp8 state entries (byte 0 first)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          f32x4 sv = e4m3x4_to_f32(raw[u][x]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[e] = fmaf(qki.y, vj[4 * x + e], sv[e]);
            acc[4 * x + e] = fmaf(qki.x, sv[e], acc[4 * x + e]);
          }
          w[x] = f32_to_e4m3x4(sv);
        }
        __builtin_nontemporal_store(w, Sh + (size_t)i * U16_PER_ROW + cg);
      }
    };
#pragma unroll 1
    for (int m0 = 0; m0 < RPL; m0 += U) rows(m0);
  } else {
    for (int m0 = 0; m0 < RPL; m0 += U) {
      u32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = rph + RP * (m0 + u);
        raw[u] = __builtin_nontemporal_load(Sh + (size_t)i * U16_PER_ROW + cg);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = rph + RP * (m0 + u);
        const float2 qki = qk[wave][i];
        u32x4 w;
        if constexpr (ST == kStBF16) {
          // each 32-bit word holds two bf16 state entries (low half first)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t word = raw[u][x];
            float s0 = __uint_as_float(word << 16);
            float s1 = __uint_as_float(word & 0xffff0000u);
            s0 = fmaf(qki.y, vj[2 * x], s0);
            s1 = fmaf(qki.y, vj[2 * x + 1], s1);
            acc[2 * x] = fmaf(qki.x, s0, acc[2 * x]);
            acc[2 * x + 1] = fmaf(qki.x, s1, acc[2 * x + 1]);
            const bf16x2 packed = {(bf16)s0, (bf16)s1};
            w[x] = __builtin_bit_cast(uint32_t, packed);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float se = fmaf(qki.y, vj[e], __uint_as_float(raw[u][e]));
            acc[e] = fmaf(qki.x, se, acc[e]);
            w[e] = __float_as_uint(se);
          }
        }
        __builtin_nontemporal_store(w, Sh + (size_t)i * U16_PER_ROW + cg);
      }
    }
  }

  // lanes with equal cg hold partial sums over disjoint rows
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], off, 64);

  if (rph == 0) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const size_t oi = (size_t)h * D + cg * VE + e;
      if constexpr (IO_BF16)
        ((u16 *)a.o)[oi] = f32_to_bf16_bits(acc[e]);
      else
        ((float *)a.o)[oi] = acc[e];
    }
  }
}

template <int D, bool IO, int ST>
hipError_t go(const DecodeArgs &a, hipStream_t stream) {
  const int64_t grid = (a.BH + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((decode_kernel<D, IO, ST>), dim3((unsigned)grid), dim3(64 * kWavesPerBlock), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool IO>
hipError_t go_st(const DecodeArgs &a, int st, hipStream_t stream) {
  switch (st) {
    case kStF32: return go<D, IO, kStF32>(a, stream);
    case kStBF16: return go<D, IO, kStBF16>(a, stream);
    case kStE4M3: return go<D, IO, kStE4M3>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t decode_launch(DecodeArgs a, int d, bool io_bf16, int state_fmt, hipStream_t stream) {
  if (d == 128) return io_bf16 ? go_st<128, true>(a, state_fmt, stream) : go_st<128, false>(a, state_fmt, stream);
  if (d == 64) return io_bf16 ? go_st<64, true>(a, state_fmt, stream) : go_st<64, false>(a, state_fmt, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
