// State accumulation over a token segment: S += K^T V, i.e. the recurrence
// S_t = S_{t-1} + k_t v_t^T of "MiniMax-M1で理解する" (zenn.dev/liushuzhi),
// section "線形アテンションの数学的基礎", applied to N tokens at once without
// reading q or producing outputs.  It is the per-segment pass of
// sequence-parallel prefill: each segment's K^T V, prefix-summed across the
// segments, is the initial state of the next segment.
//
// bf16 I/O: one workgroup (4 waves) per (sequence, 64 x 64 tile of S).  K and
// V columns of the tile stream HBM -> LDS through direct loads three tiles of
// 128 tokens deep; each wave owns 16 rows x 64 columns of the tile and
// accumulates K^T V on bf16 matrix cores with fp32 accumulation, reading both
// operands with transposing LDS reads.  The tiles of one sequence get
// workgroup ids congruent mod 8 (the same XCD), so their shared K and V
// columns can hit that XCD's L2.
//
// fp32 I/O: a plain fp32 tiled kernel of the same decomposition.
//
// Token-split variant (bf16 I/O): one workgroup per (sequence, chunk of
// tokens) accumulates the whole d x d state of its chunk, so that every K
// and V byte is read by exactly one workgroup, as whole rows (the tile
// decomposition above reads each row once per state tile row or column:
// twice per byte through L1, however well L2 serves the repeats).  The
// first chunk starts from the state; the others write their partial sums to
// a caller-provided workspace, which a second kernel adds into the state in
// chunk order.  The summation order is fixed, so results are deterministic.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lal {
namespace {

constexpr int kTile = 64;     // S tile edge (rows and columns per workgroup)
constexpr int kTok = 128;     // tokens per staged tile
constexpr int kStages = 3;    // staged tiles in flight
constexpr int kWavesSD = 4;
constexpr int kThreadsSD = kWavesSD * 64;
constexpr int kRowBytes = kTile * 2;  // one staged row: 64 bf16
constexpr int kCpr = kRowBytes / 16;  // 16-byte chunks per staged row (8)
// direct loads per staged tile and tensor: kTok rows x 128 B, 1 KiB each
constexpr int kInstPerTensor = kTok * kRowBytes / 1024;          // 16
constexpr int kInstPerWave = 2 * kInstPerTensor / kWavesSD;      // 8

// XOR swizzle of the 16-byte chunks of a staged row (8 chunks per row): makes
// the transposing reads of 16 rows x 8 bytes conflict-free.
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ u32x4 sd_desc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// Direct HBM -> LDS load, 16 bytes per lane (lane l lands at lds_base + 16 l),
// issued from inline assembly and awaited explicitly (the compiler's own
// tracking of such loads would drain them before every LDS read).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void sd_dma(u32x4 desc, int voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(desc), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void sd_wait(int n) {
  if (n == 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // kInstPerWave
}
static_assert(kInstPerWave == 8, "wait count");

__device__ __forceinline__ void sd_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D>
__global__ __launch_bounds__(kThreadsSD) void state_delta_bf16_kernel(StateDeltaArgs a) {
  constexpr int NT = D / kTile;  // tiles per S edge
  __shared__ __attribute__((aligned(1024))) u16 Ks[kStages][kTok * kTile];
  __shared__ __attribute__((aligned(1024))) u16 Vs[kStages][kTok * kTile];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;

  // workgroup -> (sequence, tile): the NT*NT tiles of one sequence share an
  // XCD when the grid is a multiple of 8 * NT * NT
  const int64_t wg = blockIdx.x;
  int64_t bh;
  int tile;
  if constexpr (NT > 1) {
    if (a.xcd_map) {
      const int64_t xcd = wg & 7, local = wg >> 3;
      tile = (int)(local % (NT * NT));
      bh = (local / (NT * NT)) * 8 + xcd;
    } else {
      bh = wg / (NT * NT);
      tile = (int)(wg % (NT * NT));
    }
  } else {
    bh = wg;
    tile = 0;
  }
  const int i0 = (tile / NT) * kTile, j0 = (tile % NT) * kTile;
  const int64_t N = a.N;
  const u16 *kh = a.k + (size_t)bh * (size_t)N * D + i0;
  const u16 *vh = a.v + (size_t)bh * (size_t)N * D + j0;
  float *Sh = a.state + (size_t)bh * D * D;

  // wave w owns S rows i0 + 16w .. +15, columns j0 .. j0+63
  f32x4 S_acc[4];
#pragma unroll
  for (int y = 0; y < 4; ++y)
#pragma unroll
    for (int e = 0; e < 4; ++e) S_acc[y][e] = Sh[(size_t)(i0 + 16 * wave + 4 * g + e) * D + j0 + 16 * y + lr];
  // consume the initial state here, so the compiler's wait for its loads
  // comes before the direct loads are issued (and does not drain them)
#pragma unroll
  for (int y = 0; y < 4; ++y) asm volatile("" ::"v"(S_acc[y]));

  const int ntile = (int)((N + kTok - 1) / kTok);
  // issue the direct loads of staged tile t (rows past N read zero)
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)t * kTok;
    const int64_t rows = N - t0 < kTok ? N - t0 : kTok;
    const uint32_t bytes = (uint32_t)((rows - 1) * D * 2 + kRowBytes);
    const u32x4 dk = sd_desc(kh + (size_t)t0 * D, bytes);
    const u32x4 dv = sd_desc(vh + (size_t)t0 * D, bytes);
    const int st = t % kStages;
#pragma unroll
    for (int m = 0; m < kInstPerWave; ++m) {
      const int inst = wave + kWavesSD * m;           // 0 .. 31: K then V
      const int ti = inst % kInstPerTensor;            // instruction within the tensor
      const int row = ti * 8 + lane / kCpr;            // 8 rows of 128 B per instruction
      const int c = swz8(row, lane % kCpr);
      const int voff = (row * D + c * 8) * 2;
      u16 *dst = (inst < kInstPerTensor ? Ks[st] : Vs[st]) + ti * 512;
      sd_dma(inst < kInstPerTensor ? dk : dv, voff,
             __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) u16 *)dst));
    }
  };

  // transposing-read offsets (bytes) of the K^T operand (this wave's 16 rows
  // of S) and of the V operand (4 column tiles), rows 4g + lr/4 of a 16-row group
  const int rr = 4 * g + (lr >> 2), h = (lr & 3) >> 1, lo8 = 8 * (lr & 1);
  const int ktr = rr * kRowBytes + (swz8(rr, 2 * wave + h) << 4) + lo8;
  int vtr[4];
#pragma unroll
  for (int y = 0; y < 4; ++y) vtr[y] = rr * kRowBytes + (swz8(rr, 2 * y + h) << 4) + lo8;

  auto ldtr = [](const u16 *base, int off0, int off1) {
    return join_tr(lds_read_tr((const u16 *)((const char *)base + off0)),
                   lds_read_tr((const u16 *)((const char *)base + off1)));
  };

  issue(0);
  if (ntile > 1) issue(1);
  for (int t = 0; t < ntile; ++t) {
    sd_wait(t + 1 < ntile ? kInstPerWave : 0);  // tile t has landed (t+1 may be in flight)
    sd_barrier();  // every wave's loads of tile t are visible; tile t-1's reads are done
    if (t + 2 < ntile) issue(t + 2);            // into the stage tile t-1 used
    const u16 *Kc = Ks[t % kStages];
    const u16 *Vc = Vs[t % kStages];
#pragma unroll
    for (int cc = 0; cc < kTok / 32; ++cc) {
      const int c0 = 32 * cc;
      const bf16x8 ka = ldtr(Kc, ktr + c0 * kRowBytes, ktr + (c0 + 16) * kRowBytes);
      bf16x8 vb[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) vb[y] = ldtr(Vc, vtr[y] + c0 * kRowBytes, vtr[y] + (c0 + 16) * kRowBytes);
#pragma unroll
      for (int y = 0; y < 4; ++y) S_acc[y] = mfma_16x16x32(ka, vb[y], S_acc[y]);
    }
  }

#pragma unroll
  for (int y = 0; y < 4; ++y)
#pragma unroll
    for (int e = 0; e < 4; ++e) Sh[(size_t)(i0 + 16 * wave + 4 * g + e) * D + j0 + 16 * y + lr] = S_acc[y][e];
}

// fp32 I/O: workgroup per (sequence, 64 x 64 tile), 256 threads, each thread
// 4 x 4 outputs; 32 tokens of K and V columns staged in LDS at a time.
template <int D>
__global__ __launch_bounds__(256) void state_delta_f32_kernel(StateDeltaF32Args a) {
  constexpr int NT = D / kTile;
  constexpr int TT = 32;
  __shared__ float Kt[TT][kTile + 1];
  __shared__ float Vt[TT][kTile + 1];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / (NT * NT);
  const int tile = (int)(blockIdx.x % (NT * NT));
  const int i0 = (tile / NT) * kTile, j0 = (tile % NT) * kTile;
  const int64_t N = a.N;
  const float *kh = a.k + (size_t)bh * (size_t)N * D;
  const float *vh = a.v + (size_t)bh * (size_t)N * D;
  float *Sh = a.state + (size_t)bh * D * D;
  const int ti = tid / 16, tj = tid % 16;  // rows 4ti.., columns 4tj..
  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = Sh[(size_t)(i0 + 4 * ti + x) * D + j0 + 4 * tj + y];
  for (int64_t t0 = 0; t0 < N; t0 += TT) {
    for (int e = tid; e < TT * kTile; e += 256) {
      const int r = e / kTile, c = e % kTile;
      const bool in = t0 + r < N;
      Kt[r][c] = in ? kh[(size_t)(t0 + r) * D + i0 + c] : 0.f;
      Vt[r][c] = in ? vh[(size_t)(t0 + r) * D + j0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < TT; ++r) {
      float kk[4], vv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) kk[x] = Kt[r][4 * ti + x];
#pragma unroll
      for (int y = 0; y < 4; ++y) vv[y] = Vt[r][4 * tj + y];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(kk[x], vv[y], acc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) Sh[(size_t)(i0 + 4 * ti + x) * D + j0 + 4 * tj + y] = acc[x][y];
}

// ---- token-split variant ----
constexpr int kSplitTok = 64;    // tokens per staged tile
constexpr int kSplitStages = 4;  // staged tiles (three in flight while one is read)

// physical 16-byte chunk of logical chunk c in staged row r (an involution;
// conflict-free transposing reads of 16 rows x 8 bytes)
template <int CPR>
__device__ __forceinline__ int swz_split(int r, int c) {
  if constexpr (CPR == 16)
    return c ^ ((r & 7) << 1);
  else
    return c ^ ((r >> 1) & 7);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// as sd_dma, non-temporal: each byte is read by one workgroup, once
__device__ __forceinline__ void sd_dma_nt(u32x4 desc, int voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voff), "s"(desc), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D>
__global__ __launch_bounds__(kThreadsSD) void state_split_bf16_kernel(StateSplitArgs a) {
  constexpr int CPR = D / 8;                     // 16-byte chunks per staged row
  constexpr int RB = D * 2;                      // bytes per staged row
  constexpr int NI = D / 16;                     // row tiles of S
  constexpr int NJW = D / 64;                    // column tiles per wave
  constexpr int RPI = 1024 / RB;                 // rows per direct load (1 KiB)
  constexpr int INST = kSplitTok / RPI;          // direct loads per tensor and stage
  constexpr int IPW = 2 * INST / kWavesSD;       // per wave and stage
  static_assert(2 * INST % kWavesSD == 0 && IPW <= 16, "direct loads per wave");
  __shared__ __attribute__((aligned(1024))) u16 Ks[kSplitStages][kSplitTok * D];
  __shared__ __attribute__((aligned(1024))) u16 Vs[kSplitStages][kSplitTok * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;

  const int64_t bh = (int64_t)blockIdx.x / a.chunks;
  const int64_t c = (int64_t)blockIdx.x % a.chunks;
  const int64_t N = a.N;
  const int64_t t_begin = c * a.chunk_len;
  const int64_t len = (N - t_begin < a.chunk_len ? N - t_begin : a.chunk_len);  // >= 1 by the host plan
  const u16 *kh = a.k + ((size_t)bh * (size_t)N + (size_t)t_begin) * D;
  const u16 *vh = a.v + ((size_t)bh * (size_t)N + (size_t)t_begin) * D;
  const bool from_state = c == 0 && !a.all_partial;
  float *out = from_state ? a.state + (size_t)bh * D * D
                          : a.partial + ((size_t)(a.all_partial ? c : c - 1) * a.BH + (size_t)bh) * D * D;

  // wave w owns S columns 16 NJW w .. + 16 NJW - 1, all rows; acc[x][y] holds
  // rows 16x + 4g + e, column 16 (NJW w + y) + lr
  f32x4 acc[NI][NJW];
#pragma unroll
  for (int x = 0; x < NI; ++x)
#pragma unroll
    for (int y = 0; y < NJW; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (from_state) {
#pragma unroll
    for (int x = 0; x < NI; ++x)
#pragma unroll
      for (int y = 0; y < NJW; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[x][y][e] = out[(size_t)(16 * x + 4 * g + e) * D + 16 * (NJW * wave + y) + lr];
  }
  // consume the initial state before the direct loads are issued, so the
  // compiler's wait for its loads does not drain them
#pragma unroll
  for (int x = 0; x < NI; ++x)
#pragma unroll
    for (int y = 0; y < NJW; ++y) asm volatile("" ::"v"(acc[x][y]));

  const int nst = (int)((len + kSplitTok - 1) / kSplitTok);
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)t * kSplitTok;
    const int64_t rows = len - t0 < kSplitTok ? len - t0 : kSplitTok;
    const uint32_t bytes = (uint32_t)(rows * RB);  // rows past the chunk read zero
    const u32x4 dk = sd_desc(kh + (size_t)t0 * D, bytes);
    const u32x4 dv = sd_desc(vh + (size_t)t0 * D, bytes);
    const int st = t % kSplitStages;
#pragma unroll
    for (int m = 0; m < IPW; ++m) {
      const int inst = wave + kWavesSD * m;  // K loads, then V loads
      const int ti = inst % INST;
      const int row = ti * RPI + lane / CPR;
      const int cc = swz_split<CPR>(row, lane % CPR);
      u16 *dst = (inst < INST ? Ks[st] : Vs[st]) + ti * 512;
      sd_dma_nt(inst < INST ? dk : dv, row * RB + cc * 16,
                __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) u16 *)dst));
    }
  };

  // transposing-read offsets: rows 4g + lr/4 of a 16-row group, columns
  // 16 tile + 4 (lr % 4) (see lds_read_tr)
  const int rr = 4 * g + (lr >> 2), h = (lr & 3) >> 1, lo8 = 8 * (lr & 1);
  auto tr_off = [&](int tile) { return rr * RB + (swz_split<CPR>(rr, 2 * tile + h) << 4) + lo8; };
  auto ldtr = [](const u16 *base, int off0, int off1) {
    return join_tr(lds_read_tr((const u16 *)((const char *)base + off0)),
                   lds_read_tr((const u16 *)((const char *)base + off1)));
  };

  issue(0);
  if (nst > 1) issue(1);
  if (nst > 2) issue(2);
  for (int t = 0; t < nst; ++t) {
    // tile t has landed once at most the loads of the tiles after it remain
    const int ahead = nst - 1 - t;
    if (ahead >= 2)
      vm_wait<2 * IPW>();
    else if (ahead == 1)
      vm_wait<IPW>();
    else
      vm_wait<0>();
    sd_barrier();  // every wave's loads of tile t are visible; tile t-1's reads are done
    if (t + 3 < nst) issue(t + 3);  // into the stage tile t-1 used
    const u16 *Kc = Ks[t % kSplitStages];
    const u16 *Vc = Vs[t % kSplitStages];
#pragma unroll
    for (int k0 = 0; k0 < kSplitTok; k0 += 32) {
      bf16x8 vb[NJW];
#pragma unroll
      for (int y = 0; y < NJW; ++y)
        vb[y] = ldtr(Vc, tr_off(NJW * wave + y) + k0 * RB, tr_off(NJW * wave + y) + (k0 + 16) * RB);
#pragma unroll
      for (int x = 0; x < NI; ++x) {
        const bf16x8 ka = ldtr(Kc, tr_off(x) + k0 * RB, tr_off(x) + (k0 + 16) * RB);
#pragma unroll
        for (int y = 0; y < NJW; ++y) acc[x][y] = mfma_16x16x32(ka, vb[y], acc[x][y]);
      }
    }
  }

#pragma unroll
  for (int x = 0; x < NI; ++x)
#pragma unroll
    for (int y = 0; y < NJW; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(size_t)(16 * x + 4 * g + e) * D + 16 * (NJW * wave + y) + lr] = acc[x][y][e];
  // the sequence's initial state, copied for the parts of a prefill cut along
  // the tokens (the final state will be written over it)
  if (a.all_partial && a.s0_copy && c == 0) {
    const f32x4 *src = (const f32x4 *)(a.state + (size_t)bh * D * D);
    f32x4 *dst = (f32x4 *)(a.s0_copy + (size_t)bh * D * D);
    for (int i = threadIdx.x; i < D * D / 4; i += kThreadsSD) dst[i] = src[i];
  }
}

// state += the partial sums of chunks 1 .. chunks-1, in chunk order; 4 values
// per thread, D*D/1024 workgroups per sequence
template <int D>
__global__ __launch_bounds__(256) void state_split_reduce_kernel(StateSplitArgs a) {
  constexpr int PER = D * D / 1024;
  const int64_t bh = blockIdx.x / PER;
  const int64_t i = (int64_t)(blockIdx.x % PER) * 256 + threadIdx.x;  // float4 index within the state
  f32x4 *st = (f32x4 *)(a.state + (size_t)bh * D * D) + i;
  f32x4 acc = *st;
  for (int64_t c = 1; c < a.chunks; ++c) acc += ((const f32x4 *)(a.partial + ((size_t)(c - 1) * a.BH + bh) * D * D))[i];
  *st = acc;
}

template <int D>
hipError_t launch_split(StateSplitArgs a, hipStream_t stream) {
  hipLaunchKernelGGL(state_split_bf16_kernel<D>, dim3((unsigned)(a.BH * a.chunks)), dim3(kThreadsSD), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.chunks == 1 || a.all_partial) return e;
  hipLaunchKernelGGL(state_split_reduce_kernel<D>, dim3((unsigned)(a.BH * (D * D / 1024))), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(StateDeltaArgs a, int64_t BH, hipStream_t stream) {
  constexpr int NT = D / kTile;
  const int64_t groups = BH * NT * NT;
  a.xcd_map = (NT > 1 && BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(state_delta_bf16_kernel<D>, dim3((unsigned)groups), dim3(kThreadsSD), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(StateDeltaF32Args a, int64_t BH, hipStream_t stream) {
  constexpr int NT = D / kTile;
  hipLaunchKernelGGL(state_delta_f32_kernel<D>, dim3((unsigned)(BH * NT * NT)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t state_delta_launch(StateDeltaArgs a, int64_t BH, int d, hipStream_t stream) {
  if (d == 128) return launch_bf16<128>(a, BH, stream);
  if (d == 64) return launch_bf16<64>(a, BH, stream);
  return hipErrorInvalidValue;
}

hipError_t state_split_launch(StateSplitArgs a, int d, hipStream_t stream) {
  if (d == 128) return launch_split<128>(a, stream);
  if (d == 64) return launch_split<64>(a, stream);
  return hipErrorInvalidValue;
}

void state_split_plan(int64_t BH, int64_t N, int cus, int64_t *chunks, int64_t *chunk_len) {
  // about one workgroup per compute unit (the kernel's 128 KiB of LDS at
  // d = 128 allows one per unit), and chunks of at least 256 tokens
  int64_t C = BH >= cus ? 1 : cus / BH;
  const int64_t cap = N / 256 > 1 ? N / 256 : 1;
  if (C > cap) C = cap;
  int64_t L = (N + C - 1) / C;
  L = (L + kSplitTok - 1) / kSplitTok * kSplitTok;
  *chunk_len = L;
  *chunks = (N + L - 1) / L;  // every chunk holds at least one token
}

hipError_t state_delta_f32_launch(StateDeltaF32Args a, int64_t BH, int d, hipStream_t stream) {
  if (d == 128) return launch_f32<128>(a, BH, stream);
  if (d == 64) return launch_f32<64>(a, BH, stream);
  return hipErrorInvalidValue;
}

}  // namespace lal
