// Several decode tokens per sequence in two steps, for verifying T <= 16
// draft tokens (speculative decoding, the open problem that "ノーフリーランチ"
// (winzheng.jp), section "推論システム統合の課題", names for linear attention):
//
//  verify:  o_t = q_t^T S_t for t = 0 .. T-1, S_t = S + sum_{s <= t} k_s v_s^T,
//           without writing the state (the recurrence of "MiniMax-M1で理解する"
//           (zenn.dev/liushuzhi), section "線形アテンションの数学的基礎",
//           unrolled over the drafts), split as
//           o_t = q_t^T S + sum_{s <= t} (q_t . k_s) v_s: one pass over the
//           state with one multiply-add per state element and draft, plus
//           the drafts' T x T table of q_t . k_s;
//  commit:  S <- S + sum_{t < a} k_t v_t^T for the a drafts accepted by the
//           sequence (a = 0 leaves S as it was: the rollback).
//
// Both are a single streaming pass over the state (read; read and write), so
// verifying T drafts costs about one decode step of state traffic instead of
// T.  Layout as in the one-token decode: two wavefronts per (batch, head),
// each walking half of its rows; each lane owns 4 columns of the rows it
// walks (16-byte fp32 or 8-byte bf16 state accesses).  verify stages q and k of the drafts in LDS (transposed,
// so a state row's multipliers are contiguous), multiplies every draft with
// no per-draft branch, and reads its columns of the drafts' v only for the
// table term; commit keeps its columns of v in registers.
//
// commit applies, per state element, the same fused multiply-adds in the
// same order as T one-token decode steps; with an fp32 state the result is
// bit-identical to them.  With a bf16 or OCP FP8 E4M3 state it rounds once,
// at the store.  Narrow states carry a per-sequence scale and are kept in
// stored units (state / scale) as in the one-token decode: verify multiplies
// the state part of its outputs by the scale, commit divides v by it.
#include <type_traits>

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

// LDS bytes per verify wave: q^T of TM drafts in fp32, k^T in the I/O type
// (it feeds only the table), and the TM x TM table of q_t . k_s
template <int D, int TM, bool IO_BF16>
constexpr size_t verify_lds_bytes() {
  return 4 * (size_t)D * TM + (IO_BF16 ? 2 : 4) * (size_t)D * TM + 4 * (size_t)TM * TM;
}

// verify, with TM >= T drafts of room.  Per state row i each lane adds
// q_t[i] S[i][cols] to output t (the state part), then the lanes build the
// table P[t][s] = q_t . k_s together and each adds sum_{s <= t} P[t][s] v_s
// for its columns (the drafts' own part).
//
// WPH waves share a head: each walks RPL / WPH of its row steps and the
// second adds its state part to the first's through LDS.
template <int D, bool IO_BF16, int ST, int TM, int WPH, int UV = 8, bool PIPE = false>
__global__ __launch_bounds__(64 * kWV) void verify_kernel(DecodeMultiArgs a) {
  constexpr int ES = ST == kStF32 ? 4 : ST == kStBF16 ? 2 : 1;
  constexpr int LPR = D / 4;    // lanes per state row (4 columns each)
  constexpr int RP = 64 / LPR;  // rows per wave access
  constexpr int RPL = D / RP;   // rows per lane
  constexpr int RW = RPL / WPH;  // row steps per wave
  constexpr int U = RW < UV ? RW : UV;  // rows per lane in one batch of loads
  constexpr int HPB = kWV / WPH;     // heads per workgroup
  static_assert(kWV % WPH == 0 && RPL % WPH == 0 && RW % U == 0, "row split");
  static_assert(TM % 4 == 0, "LDS rows of whole float4s");
  constexpr int EPC = IO_BF16 ? 8 : 4;           // elements per 16-byte piece of q or k
  constexpr int NP = (D * TM / EPC + 63) / 64;   // pieces per lane, at most
  extern __shared__ float lds[];
  const int T = a.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  using KT = std::conditional_t<IO_BF16, u16, float>;  // bf16 bits or fp32
  char *wl = (char *)lds + (size_t)wave * verify_lds_bytes<D, TM, IO_BF16>();
  float *qT = (float *)wl;                                     // qT[i * TM + t]
  KT *kT = (KT *)(wl + 4 * (size_t)D * TM);                    // kT[i * TM + t]
  float *P = (float *)(wl + (4 + sizeof(KT)) * (size_t)D * TM);  // P[t * TM + s] = q_t . k_s
  __shared__ float red[WPH > 1 ? HPB : 1][WPH > 1 ? TM * 4 : 1][LPR];  // each head's second wave's state part
  const int sub = wave % WPH;
  const int64_t h = (int64_t)blockIdx.x * HPB + wave / WPH;
  const bool valid = h < a.BH;
  const int cg = lane % LPR, rph = lane / LPR;
  const char *Sh = (const char *)a.state + (size_t)(valid ? h : 0) * D * D * ES;
  auto load_rows = [&](float(&s)[U][4], int m0) {
#pragma unroll
    for (int u = 0; u < U; ++u) ld_state4<ST>(Sh + (size_t)(rph + RP * (m0 + u)) * D * ES, cg, s[u]);
  };

  if (valid) {
    // q and k of the drafts, transposed into LDS, in groups of at most 4
    // 16-byte pieces per lane: every load of a group is issued before its
    // first store (the stores wait on them)
    const int npieces = D * T / EPC;
    const char *qb = (const char *)a.q + (size_t)h * T * D * (IO_BF16 ? 2 : 4);
    const char *kb = (const char *)a.k + (size_t)h * T * D * (IO_BF16 ? 2 : 4);
    constexpr int NG = NP < 4 ? NP : 4;
    static_assert(NP % NG == 0, "piece groups");
#pragma unroll
    for (int j0 = 0; j0 < NP; j0 += NG) {
      u32x4 qp[NG], kp[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int c = lane + 64 * (j0 + j);
        if (c < npieces) {
          qp[j] = *(const u32x4 *)(qb + (size_t)c * 16);
          kp[j] = *(const u32x4 *)(kb + (size_t)c * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int c = lane + 64 * (j0 + j);
        if (c < npieces) {
          const int t = c * EPC / D, i0 = c * EPC % D;
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            float qv;
            KT kv;
            if constexpr (IO_BF16) {
              const uint32_t wq = qp[j][e / 2], wk = kp[j][e / 2];
              qv = __uint_as_float(e & 1 ? wq & 0xffff0000u : wq << 16);
              kv = (u16)(e & 1 ? wk >> 16 : wk & 0xffffu);
            } else {
              qv = __uint_as_float(qp[j][e]);
              kv = __uint_as_float(kp[j][e]);
            }
            qT[(i0 + e) * TM + t] = qv;
            kT[(i0 + e) * TM + t] = kv;
          }
        }
      }
    }
    // q of the drafts past T reads as zero in the state pass
    if (T < TM) {
      const int rest = TM - T;
      for (int c = lane; c < D * rest; c += 64) qT[(c / rest) * TM + T + c % rest] = 0.f;
    }
  }
  __syncthreads();

  // narrow states are read in stored units: the state value is code * scale
  const float sc = (ST != kStF32 && valid && a.scale) ? a.scale[h] : 1.f;
  float acc[TM][4];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[t][e] = 0.f;

  // q of row i for all TM drafts, as TM / 4 float4 LDS reads
  auto read_q = [&](f32x4(&q)[TM / 4], int i) {
#pragma unroll
    for (int t4 = 0; t4 < TM / 4; ++t4) q[t4] = *(const f32x4 *)(qT + i * TM + 4 * t4);
  };
  // One batch of rows.  Every draft is multiplied, with no per-draft branch
  // (q of drafts t >= T is zero in LDS, and their outputs are not stored).
  // The next row's q is read while a row is multiplied, and a scheduling
  // barrier per row keeps the compiler from hoisting all rows' LDS reads
  // (which would not fit in registers).
  auto mult_rows = [&](const float(&s)[U][4], int m0) {
    f32x4 qn[TM / 4];
    read_q(qn, rph + RP * m0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 qc[TM / 4];
#pragma unroll
      for (int t4 = 0; t4 < TM / 4; ++t4) qc[t4] = qn[t4];
      if (u + 1 < U) read_q(qn, rph + RP * (m0 + u + 1));
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(qc[t / 4][t % 4], s[u][e], acc[t][e]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (valid) {
    if constexpr (PIPE) {
      // the loads of batch b + 1 are in flight while batch b is multiplied
      float cur[U][4], nxt[U][4];
      load_rows(cur, sub * RW);
#pragma unroll
      for (int m0 = sub * RW; m0 < (sub + 1) * RW; m0 += U) {
        if (m0 + U < (sub + 1) * RW) load_rows(nxt, m0 + U);
        mult_rows(cur, m0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) cur[u][e] = nxt[u][e];
      }
    } else {
#pragma unroll 1
      for (int m0 = sub * RW; m0 < (sub + 1) * RW; m0 += U) {
        float s[U][4];
        load_rows(s, m0);
        mult_rows(s, m0);
      }
    }
  }
  // lanes with equal cg hold partial sums over disjoint rows
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int t = 0; t < TM; ++t)
      if (t < T)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] += __shfl_xor(acc[t][e], off, 64);
  if constexpr (WPH > 1) {
    // the waves of a head add their state parts in wave order
    if (sub == 1 && rph == 0) {
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave / WPH][4 * t + e][cg] = acc[t][e];
    }
    __syncthreads();
    if (sub != 0) return;
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] += red[wave / WPH][4 * t + e][cg];
  }
  if (!valid) return;

  // this lane's 4 columns of every draft's v, needed only from here on (the
  // state pass runs without them, with fewer registers); their loads are in
  // flight while the table below is built
  float vr[TM][4];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const size_t base = ((size_t)h * T + t) * D + 4 * cg;
    if (t < T) {
      if constexpr (IO_BF16) {
        const u32x2 w = *(const u32x2 *)((const u16 *)a.v + base);
        vr[t][0] = __uint_as_float(w[0] << 16);
        vr[t][1] = __uint_as_float(w[0] & 0xffff0000u);
        vr[t][2] = __uint_as_float(w[1] << 16);
        vr[t][3] = __uint_as_float(w[1] & 0xffff0000u);
      } else {
        const f32x4 w = *(const f32x4 *)((const float *)a.v + base);
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[t][e] = w[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) vr[t][e] = 0.f;
    }
  }

  // P[t][s] = q_t . k_s.  Lane l takes pair group g = l % G (draft t and
  // drafts s0 .. s0 + 3) over row slice l / G; the slices are summed across
  // lanes.  Entries with t or s >= T are never read.
  {
    constexpr int G = TM * TM / 4, NS = 64 / G, RS = D / NS;
    static_assert(64 % G == 0 && D % NS == 0, "pair groups");
    const int g = lane % G, sl = lane / G, tq = g / (TM / 4), s0 = 4 * (g % (TM / 4));
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int i = sl * RS; i < (sl + 1) * RS; ++i) {
      const float qi = qT[i * TM + tq];
      f32x4 k4;
      if constexpr (IO_BF16) {
        const u32x2 w = *(const u32x2 *)(kT + i * TM + s0);
        k4 = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                   __uint_as_float(w[1] & 0xffff0000u)};
      } else {
        k4 = *(const f32x4 *)(kT + i * TM + s0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = fmaf(qi, k4[e], p[e]);
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] += __shfl_xor(p[e], off, 64);
    if (sl == 0) *(f32x4 *)(P + tq * TM + s0) = p;
  }
  // the table was written by other lanes of this wave: LDS accesses complete
  // before it is read
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();

  // o_t = scale * (q_t^T S) + sum_{s <= t} P[t][s] v_s
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < T) {
      float pr[TM];
#pragma unroll
      for (int s4 = 0; s4 < TM; s4 += 4) {
        const f32x4 p4 = *(const f32x4 *)(P + t * TM + s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[s4 + e] = p4[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = ST == kStF32 ? acc[t][e] : acc[t][e] * sc;
#pragma unroll
      for (int s = 0; s <= t; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(pr[s], vr[s][e], acc[t][e]);
    }
  }

  if (rph == 0) {
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < T) {
        const size_t oi = ((size_t)h * T + t) * D + 4 * cg;
        if constexpr (IO_BF16) {
          const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[t][0]) | ((uint32_t)f32_to_bf16_bits(acc[t][1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_bits(acc[t][2]) | ((uint32_t)f32_to_bf16_bits(acc[t][3]) << 16);
          *(u32x2 *)((u16 *)a.o + oi) = u32x2{lo, hi};
        } else {
          *(f32x4 *)((float *)a.o + oi) = f32x4{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
        }
      }
    }
  }
}

// commit, with TM >= T drafts of room: per state element, the accepted
// drafts' updates in draft order, the fused multiply-adds of as many
// one-token decode steps.  k of the drafts is staged in LDS (transposed,
// fp32) with 16-byte loads, each group issued before its stores; each lane keeps its
// 4 columns of the accepted drafts' v in registers.  The pass is bound by
// the state bytes in flight, so each variant asks the compiler for the
// occupancy its registers allow without spills (8, 6 and 3 waves per SIMD
// with room for 4, 8 and 16 drafts).
constexpr int commit_waves_per_simd(int TM) { return TM <= 4 ? 8 : TM <= 8 ? 6 : 3; }

//
// WPH waves share a head, each updating RPL / WPH of its row steps (each
// stages the drafts' k itself); with PIPE the loads of the next batch of U
// rows are in flight while a batch is updated.
template <int D, bool IO_BF16, int ST, int TM, int WPH, int U, bool PIPE>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(commit_waves_per_simd(TM))))
void commit_kernel(DecodeMultiArgs a) {
  constexpr int ES = ST == kStF32 ? 4 : ST == kStBF16 ? 2 : 1;
  constexpr int LPR = D / 4;
  constexpr int RP = 64 / LPR;
  constexpr int RPL = D / RP;
  constexpr int RW = RPL / WPH;  // row steps per wave
  constexpr int HPB = kW / WPH;  // heads per workgroup
  static_assert(kW % WPH == 0 && RPL % WPH == 0 && RW % U == 0, "row split");
  static_assert(TM % 4 == 0, "LDS rows of whole float4s");
  constexpr int EPC = IO_BF16 ? 8 : 4;          // elements per 16-byte piece of k
  constexpr int NP = (D * TM / EPC + 63) / 64;  // pieces per lane, at most
  extern __shared__ float lds[];
  const int T = a.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float *kT = lds + (size_t)wave * D * TM;  // kT[i * TM + t]
  const int sub = wave % WPH;
  const int64_t h = (int64_t)blockIdx.x * HPB + wave / WPH;
  const bool valid = h < a.BH;
  int cnt = 0;
  if (valid) {
    cnt = a.accept ? a.accept[h / a.H] : T;
    cnt = cnt < 0 ? 0 : (cnt > T ? T : cnt);
    const int npieces = D * T / EPC;
    const char *kb = (const char *)a.k + (size_t)h * T * D * (IO_BF16 ? 2 : 4);
    constexpr int NG = NP < 4 ? NP : 4;  // pieces per group
    static_assert(NP % NG == 0, "piece groups");
#pragma unroll
    for (int j0 = 0; j0 < NP; j0 += NG) {
      u32x4 kp[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int c = lane + 64 * (j0 + j);
        if (c < npieces) kp[j] = *(const u32x4 *)(kb + (size_t)c * 16);
      }
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int c = lane + 64 * (j0 + j);
        if (c < npieces) {
          const int t = c * EPC / D, i0 = c * EPC % D;
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            if constexpr (IO_BF16) {
              const uint32_t w = kp[j][e / 2];
              kT[(i0 + e) * TM + t] = __uint_as_float(e & 1 ? w & 0xffff0000u : w << 16);
            } else {
              kT[(i0 + e) * TM + t] = __uint_as_float(kp[j][e]);
            }
          }
        }
      }
    }
  }
  __syncthreads();
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if (!valid || cnt == 0) return;

  const int cg = lane % LPR, rph = lane / LPR;
  // narrow states are updated in stored units: v / scale
  const float inv = (ST != kStF32 && a.scale) ? 1.f / a.scale[h] : 1.f;
  float vr[TM][4];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const size_t base = ((size_t)h * T + t) * D + 4 * cg;
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < cnt) {
      if constexpr (IO_BF16) {
        const u32x2 x = *(const u32x2 *)((const u16 *)a.v + base);
        w[0] = __uint_as_float(x[0] << 16);
        w[1] = __uint_as_float(x[0] & 0xffff0000u);
        w[2] = __uint_as_float(x[1] << 16);
        w[3] = __uint_as_float(x[1] & 0xffff0000u);
      } else {
        const f32x4 x = *(const f32x4 *)((const float *)a.v + base);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = x[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) vr[t][e] = w[e] * inv;
  }

  char *Sh = (char *)a.state + (size_t)h * D * D * ES;
  auto row_of = [&](int m) { return Sh + (size_t)(rph + RP * m) * D * ES; };
  auto update = [&](int m, float(&s)[4]) __attribute__((always_inline)) {
    const int i = rph + RP * m;
    f32x4 k4[TM / 4];
#pragma unroll
    for (int t4 = 0; t4 < TM / 4; ++t4) k4[t4] = *(const f32x4 *)(kT + i * TM + 4 * t4);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < cnt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = fmaf(k4[t / 4][t % 4], vr[t][e], s[e]);
      }
    }
    st_state4<ST>(row_of(m), cg, s);
  };
  const int m_lo = sub * RW;
  if constexpr (PIPE) {
    float cur[U][4], nxt[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) ld_state4<ST>(row_of(m_lo + u), cg, cur[u]);
#pragma unroll
    for (int m0 = 0; m0 < RW; m0 += U) {
      if (m0 + U < RW) {
#pragma unroll
        for (int u = 0; u < U; ++u) ld_state4<ST>(row_of(m_lo + m0 + U + u), cg, nxt[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) update(m_lo + m0 + u, cur[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[u][e] = nxt[u][e];
    }
  } else {
    for (int m0 = 0; m0 < RW; m0 += U) {
      float s[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) ld_state4<ST>(row_of(m_lo + m0 + u), cg, s[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) update(m_lo + m0 + u, s[u]);
    }
  }
}

// Waves per head, rows per lane in a batch and pipelining, per state format.
// Measured at 256 x 64 sequences, d = 128, 4 drafts (0-4 accepted), bf16
// I/O, against one wave per head with unpipelined 8-row batches; states and
// fp32-state outputs bitwise the same:
//  * commit, fp32 state: 2 waves, pipelined 4-row batches: 0.300 ms against
//    0.329 (one wave pipelined: 0.322; 2 waves unpipelined 8 rows: 0.312);
//  * commit, bf16 state: 2 waves, pipelined 4-row batches: 0.154 ms against
//    0.160 (one wave pipelined 8 rows: 0.159);
//  * commit, E4M3 state: 2 waves, one batch of 8 rows: 0.080 ms against 0.086;
//  * verify: 2 waves, and for an fp32 state with room for 4 drafts pipelined
//    16-row batches: 0.175 ms against 0.184 (unpipelined 8 rows: 0.181;
//    pipelined 8 rows: 0.178); bf16 state, unpipelined 8 rows: 0.097 ms
//    against 0.098 (pipelined 8 or 16 rows: 0.098, 0.103).
template <int ST>
struct CommitTune {
  static constexpr int WPH = 2;
  static constexpr int UMAX = ST == kStE4M3 ? 8 : 4;
  static constexpr bool PIPE = ST != kStE4M3;
};
template <int ST, int TM>
struct VerifyTune {
  static constexpr int WPH = 2;
  static constexpr bool PIPE = ST == kStF32 && TM <= 4;  // registers for two batches
  static constexpr int UV = PIPE ? 16 : 8;
};

template <int D, bool IO, int ST, int TM>
void commit_go(const DecodeMultiArgs &a, hipStream_t stream) {
  using C = CommitTune<ST>;
  constexpr int RW = D / (64 / (D / 4)) / C::WPH;
  constexpr int U = RW < C::UMAX ? RW : C::UMAX;
  constexpr int HPB = kW / C::WPH;
  const int64_t grid = (a.BH + HPB - 1) / HPB;
  // LDS: kW * D * TM floats, <= 32 KiB
  hipLaunchKernelGGL((commit_kernel<D, IO, ST, TM, C::WPH, U, C::PIPE>), dim3((unsigned)grid), dim3(64 * kW),
                     (size_t)kW * D * TM * sizeof(float), stream, a);
}

template <int D, bool IO, int ST, int TM>
void verify_go(const DecodeMultiArgs &a, hipStream_t stream) {
  using V = VerifyTune<ST, TM>;
  constexpr int HPB = kWV / V::WPH;
  const int64_t grid = (a.BH + HPB - 1) / HPB;
  // LDS scales with TM: 26 KiB at d = 128, bf16 I/O and TM = 16
  const size_t lds = (size_t)kWV * verify_lds_bytes<D, TM, IO>();
  hipLaunchKernelGGL((verify_kernel<D, IO, ST, TM, V::WPH, V::UV, V::PIPE>), dim3((unsigned)grid), dim3(64 * kWV), lds,
                     stream, a);
}

template <int D, bool IO, int ST>
hipError_t go(const DecodeMultiArgs &a, bool commit, hipStream_t stream) {
  // room for TM = 4, 8 or 16 drafts (registers and LDS scale with it)
  if (commit) {
    if (a.T <= 4) commit_go<D, IO, ST, 4>(a, stream);
    else if (a.T <= 8) commit_go<D, IO, ST, 8>(a, stream);
    else commit_go<D, IO, ST, 16>(a, stream);
  } else {
    if (a.T <= 4) verify_go<D, IO, ST, 4>(a, stream);
    else if (a.T <= 8) verify_go<D, IO, ST, 8>(a, stream);
    else verify_go<D, IO, ST, 16>(a, stream);
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
