// C ABI of the linear-attention library: argument validation and dispatch.
// The operation and the conventions are documented in include/lin_attn.h.
//
// Every check that can reject a call runs on the host before the first HIP
// call, so invalid arguments never reach the device.
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <random>

#include "kernels.hpp"
#include "lin_attn.h"

// Fixed device memory of lin_attn_prefill_seqsplit_noalloc: one copy per
// device, held from the library's load until the process ends.  In host code
// the name is a host-side stand-in, not a device address: the address of each
// device's copy comes from hipGetSymbolAddress (scratch_ptr below), and only
// that address is passed to kernels.
constexpr int64_t kScratchBytes = 56ll << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool ok_ptr(const void *p) { return p != nullptr && aligned16(p); }

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

// Number of compute units of the current device, cached per device ordinal.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LIN_ATTN_EHIP;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return LIN_ATTN_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return LIN_ATTN_EHIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *out = c;
  return LIN_ATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? LIN_ATTN_OK : LIN_ATTN_EHIP; }

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on each device and cached.
int scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LIN_ATTN_EHIP;
  if (dev >= 0 && dev < kMaxDevices) {
    void *p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) {
      *out = p;
      return LIN_ATTN_OK;
    }
  }
  void *p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LIN_ATTN_EHIP;
  if (dev >= 0 && dev < kMaxDevices) g_scratch_ptr[dev].store(p, std::memory_order_relaxed);
  *out = p;
  return LIN_ATTN_OK;
}

}  // namespace

namespace {

// Shared by the prefill entry points: validation order and dispatch.
// state: fp32 state (lp_fmt == kStF32), else lp_state holds codes of
// state / lp_scale in the narrow format lp_fmt (bf16 I/O only).
int prefill_impl(const void *q, const void *k, const void *v, void *o, float *state, float *snap,
                 int64_t every, int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                 lin_attn_dtype_t io_dtype, int64_t split, void *stream, int lp_fmt = lal::kStF32,
                 void *lp_state = nullptr, const float *lp_scale = nullptr, int lp_round = 0) {
  if (B < 0 || H < 0 || N < 0 || d < 0 || block < 0 || split < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  const bool bf16 = io_dtype == LIN_ATTN_BF16;
  const int max_block = bf16 ? lal::prefill_bf16_max_block((int)d) : lal::prefill_f32_max_block((int)d);
  if (block < 16 || block > max_block || block % 16 != 0) return LIN_ATTN_EUNSUPPORTED;
  if (split != 0) {
    if (!bf16 && split != 1) return LIN_ATTN_EUNSUPPORTED;
    if (bf16 && (split > lal::prefill_bf16_max_split((int)d) || (split & (split - 1)) != 0))
      return LIN_ATTN_EUNSUPPORTED;
  }
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &total) || !mul_ok(total, d, &total)) return LIN_ATTN_EINVAL;
  // snapshots (every > 0): (N / block) / every of them per sequence
  if (every < 0 || every > 0x7fffffff) return LIN_ATTN_EINVAL;
  const int64_t nsnap = every > 0 ? (N / block) / every : 0;
  int64_t snap_elems;
  if (!mul_ok(BH, nsnap, &snap_elems) || !mul_ok(snap_elems, d * d, &snap_elems)) return LIN_ATTN_EINVAL;
  if (BH == 0 || N == 0) return LIN_ATTN_OK;
  const bool narrow = lp_fmt != lal::kStF32;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(narrow ? lp_state : (const void *)state))
    return LIN_ATTN_EINVAL;
  if (narrow && lp_scale && ((uintptr_t)lp_scale & 3)) return LIN_ATTN_EINVAL;
  if (nsnap > 0 && !ok_ptr(snap)) return LIN_ATTN_EINVAL;
  float *snap_k = nsnap > 0 ? snap : nullptr;
  hipStream_t s = (hipStream_t)stream;

  if (!bf16) {
    if (narrow) return LIN_ATTN_EUNSUPPORTED;
    if (BH > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
    lal::PrefillF32Args a{(const float *)q, (const float *)k, (const float *)v, (float *)o, state, N,
                          (int)block, snap_k, (int)every};
    return from_hip(lal::prefill_f32_launch(a, BH, (int)d, s));
  }

  int nsplit = (int)split;
  if (nsplit == 0) {
    // Enough workgroups to give every compute unit one sequence slice: split
    // the value columns of each sequence while B*H alone leaves CUs idle.
    int cus = 0;
    const int rc = cu_count(&cus);
    if (rc != LIN_ATTN_OK) return rc;
    nsplit = 1;
    while (nsplit < lal::prefill_bf16_max_split((int)d) && BH * nsplit < cus) nsplit *= 2;
  }
  if (BH * nsplit > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  if (N / block > 0x7ffffff0) return LIN_ATTN_EUNSUPPORTED;  // 32-bit block indices
  lal::PrefillArgs a{(const unsigned short *)q, (const unsigned short *)k, (const unsigned short *)v,
                     (unsigned short *)o, state, N, (int)block, nsplit, 0, snap_k, (int)every,
                     lp_state, lp_scale, lp_round};
  if (narrow) return from_hip(lal::prefill_bf16_scaled_launch(a, BH, (int)d, lp_fmt, s));
  return from_hip(lal::prefill_bf16_launch(a, BH, (int)d, s));
}

}  // namespace

extern "C" {

int lin_attn_prefill_ex(const void *q, const void *k, const void *v, void *o, float *state,
                        int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                        lin_attn_dtype_t io_dtype, int64_t split, void *stream) {
  return prefill_impl(q, k, v, o, state, nullptr, 0, B, H, N, d, block, io_dtype, split, stream);
}

int lin_attn_prefill_snapshots(const void *q, const void *k, const void *v, void *o, float *state,
                               float *snapshots, int64_t B, int64_t H, int64_t N, int64_t d,
                               int64_t block, int64_t every, lin_attn_dtype_t io_dtype, void *stream) {
  if (every < 1) return LIN_ATTN_EINVAL;
  return prefill_impl(q, k, v, o, state, snapshots, every, B, H, N, d, block, io_dtype, 0, stream);
}

int lin_attn_prefill_scaled(const void *q, const void *k, const void *v, void *o, void *state,
                            const float *state_scale, int64_t B, int64_t H, int64_t N, int64_t d,
                            int64_t block, lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype,
                            int64_t round_carry, void *stream) {
  if (round_carry != 0 && round_carry != 1) return LIN_ATTN_EINVAL;
  if (state_dtype != LIN_ATTN_BF16 && state_dtype != LIN_ATTN_FP8_E4M3) return LIN_ATTN_EUNSUPPORTED;
  if (io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;  // narrow states: bf16 I/O kernel only
  return prefill_impl(q, k, v, o, nullptr, nullptr, 0, B, H, N, d, block, io_dtype, 0, stream,
                      state_dtype == LIN_ATTN_BF16 ? lal::kStBF16 : lal::kStE4M3, state, state_scale,
                      (int)round_carry);
}

namespace {

int backward_impl(const void *q, const void *k, const void *v, const void *dout, const float *state0,
                  const float *dstate, void *dq, void *dk, void *dv, float *dstate0, int64_t B, int64_t H,
                  int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype, int64_t strategy, void *stream) {
  if (B < 0 || H < 0 || N < 0 || d < 0 || block < 0) return LIN_ATTN_EINVAL;
  if (strategy < LIN_ATTN_BWD_AUTO || strategy > LIN_ATTN_BWD_FUSED) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_BF16 && io_dtype != LIN_ATTN_F32) return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  const bool f32 = io_dtype == LIN_ATTN_F32;
  const int max_block = f32 ? lal::prefill_f32_max_block((int)d) : lal::prefill_bf16_max_block((int)d);
  if (block < 16 || block > max_block || block % 16 != 0) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &total) || !mul_ok(total, d, &total) || !mul_ok(BH, d * d, &total))
    return LIN_ATTN_EINVAL;
  if (BH == 0) return LIN_ATTN_OK;
  if ((state0 && !ok_ptr(state0)) || (dstate && !ok_ptr(dstate)) || (dstate0 && !ok_ptr(dstate0)))
    return LIN_ATTN_EINVAL;
  if (N > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(dout) || !ok_ptr(dq) || !ok_ptr(dk) ||
                !ok_ptr(dv)))
    return LIN_ATTN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0 && !dstate0) return LIN_ATTN_OK;
  if (f32) {
    // fp32 I/O: the three passes on the fp32 kernel (the strategies of the
    // bf16 path concern its matrix-core kernel; here they all run this way)
    if (BH > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
    using fp = const float *;
    lal::PrefillF32Args f{};
    f.N = N;
    f.blk = (int)block;
    f.grad = 1;
    // dV: reversed prefill of (K, Q, dout) from dS_N, ending in dS_0
    f.q = (fp)k; f.k = (fp)q; f.v = (fp)dout; f.o = (float *)dv;
    f.rev = 1; f.g_in = dstate; f.g_in_t = 0; f.g_out = dstate0;
    hipError_t e = lal::prefill_f32_launch(f, BH, (int)d, s);
    if (e != hipSuccess || N == 0) return from_hip(e);
    // dK: reversed prefill of (V, dout, Q) from dS_N^T
    f.q = (fp)v; f.k = (fp)dout; f.v = (fp)q; f.o = (float *)dk;
    f.rev = 1; f.g_in = dstate; f.g_in_t = 1; f.g_out = nullptr;
    e = lal::prefill_f32_launch(f, BH, (int)d, s);
    if (e != hipSuccess) return from_hip(e);
    // dQ: forward prefill of (dout, V, K) from S_0^T
    f.q = (fp)dout; f.k = (fp)v; f.v = (fp)k; f.o = (float *)dq;
    f.rev = 0; f.g_in = state0; f.g_in_t = 1; f.g_out = nullptr;
    return from_hip(lal::prefill_f32_launch(f, BH, (int)d, s));
  }
  int cus = 0;
  const int rc = cu_count(&cus);
  if (rc != LIN_ATTN_OK) return rc;
  int nsplit = 1;
  while (nsplit < lal::prefill_bf16_max_split((int)d) && BH * nsplit < cus) nsplit *= 2;
  // auto: the fused dK/dV sweep when the sequences fill the GPU without a
  // value split, else separate passes with the split
  const int64_t strat = strategy != LIN_ATTN_BWD_AUTO ? strategy
                        : (nsplit == 1 ? LIN_ATTN_BWD_FUSED : LIN_ATTN_BWD_SEPARATE);
  if (strat != LIN_ATTN_BWD_SEPARATE) nsplit = 1;
  if (BH * 2 * nsplit > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  if (N / block > 0x7ffffff0) return LIN_ATTN_EUNSUPPORTED;
  using u16p = const unsigned short *;
  lal::PrefillArgs a{};
  a.N = N;
  a.blk = (int)block;
  a.nsplit = nsplit;
  hipError_t e;
  if (N > 0 && strat == LIN_ATTN_BWD_FUSED) {
    // dK and dV in one reversed sweep: q and dout tiles staged once, the k
    // rows (dV role) and v rows (dK role) as queries, G from dS_N to dS_0
    a.q = (u16p)k; a.k = (u16p)q; a.v = (u16p)dout; a.o = (unsigned short *)dv;
    a.q2 = (u16p)v; a.o2 = (unsigned short *)dk;
    a.g_in = dstate; a.g_in_t = 0; a.g_out = dstate0;
    e = lal::prefill_bf16_grad_fused_launch(a, BH, (int)d, s);
  } else if (N > 0 && strat == LIN_ATTN_BWD_PAIRED) {
    // dV and dK in one launch: dK is the reversed prefill of (V, dout, Q)
    // from dS_N^T, whose keys and values are dV's values and keys, so the two
    // workgroups of a sequence stream the same Q and dout tiles
    a.q = (u16p)k; a.k = (u16p)q; a.v = (u16p)dout; a.o = (unsigned short *)dv;
    a.g_in = dstate; a.g_in_t = 0; a.g_out = dstate0;
    a.q2 = (u16p)v; a.k2 = (u16p)dout; a.v2 = (u16p)q; a.o2 = (unsigned short *)dk;
    a.g_in2 = dstate; a.g_in_t2 = 1; a.g_out2 = nullptr;
    e = lal::prefill_bf16_grad_pair_launch(a, BH, (int)d, s);
  } else {
    // dV: reversed prefill of (K, Q, dout) from dS_N; it ends in dS_0 (with no
    // tokens it only copies dS_N, or zeros, into dS_0)
    a.q = (u16p)k; a.k = (u16p)q; a.v = (u16p)dout; a.o = (unsigned short *)dv;
    a.g_in = dstate; a.g_in_t = 0; a.g_out = dstate0;
    e = lal::prefill_bf16_grad_launch(a, BH, (int)d, true, s);
    if (e != hipSuccess || N == 0) return from_hip(e);
    // dK: reversed prefill of (V, dout, Q) from dS_N^T
    a.q = (u16p)v; a.k = (u16p)dout; a.v = (u16p)q; a.o = (unsigned short *)dk;
    a.g_in = dstate; a.g_in_t = 1; a.g_out = nullptr;
    e = lal::prefill_bf16_grad_launch(a, BH, (int)d, true, s);
  }
  if (e != hipSuccess) return from_hip(e);
  // dQ: forward prefill of (dout, V, K) from S_0^T; its final state is not needed
  a = lal::PrefillArgs{};
  a.N = N;
  a.blk = (int)block;
  a.nsplit = nsplit;
  a.q = (u16p)dout; a.k = (u16p)v; a.v = (u16p)k; a.o = (unsigned short *)dq;
  a.g_in = state0; a.g_in_t = 1; a.g_out = nullptr;
  return from_hip(lal::prefill_bf16_grad_launch(a, BH, (int)d, false, s));
}

}  // namespace

int lin_attn_backward(const void *q, const void *k, const void *v, const void *dout, const float *state0,
                      const float *dstate, void *dq, void *dk, void *dv, float *dstate0, int64_t B,
                      int64_t H, int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype,
                      void *stream) {
  return backward_impl(q, k, v, dout, state0, dstate, dq, dk, dv, dstate0, B, H, N, d, block, io_dtype,
                       LIN_ATTN_BWD_AUTO, stream);
}

int lin_attn_backward_ex(const void *q, const void *k, const void *v, const void *dout, const float *state0,
                         const float *dstate, void *dq, void *dk, void *dv, float *dstate0, int64_t B,
                         int64_t H, int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype,
                         int64_t strategy, void *stream) {
  return backward_impl(q, k, v, dout, state0, dstate, dq, dk, dv, dstate0, B, H, N, d, block, io_dtype,
                       strategy, stream);
}

int lin_attn_prefill(const void *q, const void *k, const void *v, void *o, float *state, int64_t B,
                     int64_t H, int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype,
                     void *stream) {
  return lin_attn_prefill_ex(q, k, v, o, state, B, H, N, d, block, io_dtype, 0, stream);
}

namespace {
int state_fmt_of(lin_attn_dtype_t t) {
  return t == LIN_ATTN_F32 ? lal::kStF32 : t == LIN_ATTN_BF16 ? lal::kStBF16 : lal::kStE4M3;
}

int decode_impl(const void *q, const void *k, const void *v, void *o, void *state, const float *scale,
                int64_t B, int64_t H, int64_t d, lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype,
                void *stream) {
  if (B < 0 || H < 0 || d < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (state_dtype != LIN_ATTN_F32 && state_dtype != LIN_ATTN_BF16 && state_dtype != LIN_ATTN_FP8_E4M3)
    return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, d * d, &total)) return LIN_ATTN_EINVAL;
  if (BH == 0) return LIN_ATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(state)) return LIN_ATTN_EINVAL;
  if (scale && ((uintptr_t)scale & 3)) return LIN_ATTN_EINVAL;
  if ((BH + 3) / 4 > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  lal::DecodeArgs a{q, k, v, o, state, BH, scale};
  return from_hip(lal::decode_launch(a, (int)d, io_dtype == LIN_ATTN_BF16, state_fmt_of(state_dtype),
                                     (hipStream_t)stream));
}
}  // namespace

int lin_attn_decode(const void *q, const void *k, const void *v, void *o, void *state, int64_t B,
                    int64_t H, int64_t d, lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype,
                    void *stream) {
  return decode_impl(q, k, v, o, state, nullptr, B, H, d, io_dtype, state_dtype, stream);
}

int lin_attn_decode_scaled(const void *q, const void *k, const void *v, void *o, void *state,
                           const float *state_scale, int64_t B, int64_t H, int64_t d,
                           lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream) {
  if (state_dtype == LIN_ATTN_F32) return LIN_ATTN_EUNSUPPORTED;
  return decode_impl(q, k, v, o, state, state_scale, B, H, d, io_dtype, state_dtype, stream);
}

int lin_attn_prefill_recurrent(const void *q, const void *k, const void *v, void *o, float *state,
                               int64_t B, int64_t H, int64_t N, int64_t d, lin_attn_dtype_t io_dtype,
                               void *stream) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &total) || !mul_ok(total, d, &total)) return LIN_ATTN_EINVAL;
  if (BH == 0 || N == 0) return LIN_ATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(state)) return LIN_ATTN_EINVAL;
  if (BH * (d / 16) > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  int cus = 0;
  const int rc = cu_count(&cus);
  if (rc != LIN_ATTN_OK) return rc;
  lal::RecurrentArgs a{q, k, v, o, state, BH, N};
  return from_hip(lal::recurrent_launch(a, (int)d, io_dtype == LIN_ATTN_BF16, cus, (hipStream_t)stream));
}

namespace {
int decode_multi_impl(const void *q, const void *k, const void *v, void *o, void *state, const int32_t *accept,
                      bool commit, int64_t B, int64_t H, int64_t T, int64_t d, lin_attn_dtype_t io_dtype,
                      lin_attn_dtype_t state_dtype, void *stream, const float *scale = nullptr) {
  if (B < 0 || H < 0 || T < 0 || d < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (state_dtype != LIN_ATTN_F32 && state_dtype != LIN_ATTN_BF16 && state_dtype != LIN_ATTN_FP8_E4M3)
    return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  if (T > lal::decode_multi_max_tokens()) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, d * d, &total) || !mul_ok(BH, T * d, &total)) return LIN_ATTN_EINVAL;
  if (BH == 0 || T == 0) return LIN_ATTN_OK;
  if ((!commit && (!ok_ptr(q) || !ok_ptr(o))) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(state))
    return LIN_ATTN_EINVAL;
  if (accept != nullptr && ((uintptr_t)accept & 3u) != 0) return LIN_ATTN_EINVAL;
  if (scale != nullptr && ((uintptr_t)scale & 3u) != 0) return LIN_ATTN_EINVAL;
  if ((BH + 1) / 2 > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  lal::DecodeMultiArgs a{q, k, v, o, state, accept, BH, H, (int)T, scale};
  return from_hip(lal::decode_multi_launch(a, (int)d, commit, io_dtype == LIN_ATTN_BF16, state_fmt_of(state_dtype),
                                           (hipStream_t)stream));
}
}  // namespace

int lin_attn_decode_verify_scaled(const void *q, const void *k, const void *v, void *o, const void *state,
                                  const float *state_scale, int64_t B, int64_t H, int64_t T, int64_t d,
                                  lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream) {
  if (state_dtype == LIN_ATTN_F32) return LIN_ATTN_EUNSUPPORTED;
  return decode_multi_impl(q, k, v, o, const_cast<void *>(state), nullptr, false, B, H, T, d, io_dtype,
                           state_dtype, stream, state_scale);
}

int lin_attn_decode_commit_scaled(const void *k, const void *v, void *state, const float *state_scale,
                                  const int32_t *accept, int64_t B, int64_t H, int64_t T, int64_t d,
                                  lin_attn_dtype_t io_dtype, lin_attn_dtype_t state_dtype, void *stream) {
  if (state_dtype == LIN_ATTN_F32) return LIN_ATTN_EUNSUPPORTED;
  return decode_multi_impl(nullptr, k, v, nullptr, state, accept, true, B, H, T, d, io_dtype, state_dtype,
                           stream, state_scale);
}

int lin_attn_decode_verify(const void *q, const void *k, const void *v, void *o, const void *state, int64_t B,
                           int64_t H, int64_t T, int64_t d, lin_attn_dtype_t io_dtype,
                           lin_attn_dtype_t state_dtype, void *stream) {
  return decode_multi_impl(q, k, v, o, const_cast<void *>(state), nullptr, false, B, H, T, d, io_dtype,
                           state_dtype, stream);
}

int lin_attn_decode_commit(const void *k, const void *v, void *state, const int32_t *accept, int64_t B,
                           int64_t H, int64_t T, int64_t d, lin_attn_dtype_t io_dtype,
                           lin_attn_dtype_t state_dtype, void *stream) {
  return decode_multi_impl(nullptr, k, v, nullptr, state, accept, true, B, H, T, d, io_dtype, state_dtype,
                           stream);
}

int lin_attn_state_accumulate(const void *k, const void *v, float *state, int64_t B, int64_t H, int64_t N,
                              int64_t d, lin_attn_dtype_t io_dtype, void *stream) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &total) || !mul_ok(total, d, &total)) return LIN_ATTN_EINVAL;
  if (BH == 0 || N == 0) return LIN_ATTN_OK;
  if (!ok_ptr(k) || !ok_ptr(v) || !ok_ptr(state)) return LIN_ATTN_EINVAL;
  const int64_t tiles = (d / 64) * (d / 64);
  if (BH * tiles > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  // 32-bit descriptor ranges: one staged tile of 128 tokens spans < 2^31 bytes
  hipStream_t s = (hipStream_t)stream;
  if (io_dtype == LIN_ATTN_BF16) {
    lal::StateDeltaArgs a{(const unsigned short *)k, (const unsigned short *)v, state, N, 0};
    return from_hip(lal::state_delta_launch(a, BH, (int)d, s));
  }
  lal::StateDeltaF32Args a{(const float *)k, (const float *)v, state, N};
  return from_hip(lal::state_delta_f32_launch(a, BH, (int)d, s));
}

namespace {

// Validation shared by the split state accumulation and its workspace query:
// LIN_ATTN_OK with BH and the workspace bytes set, or an error code.
int split_check(int64_t B, int64_t H, int64_t N, int64_t d, lin_attn_dtype_t io_dtype, int64_t *BH_out,
                int64_t *chunks, int64_t *chunk_len, int64_t *ws_bytes) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &total) || !mul_ok(total, d, &total)) return LIN_ATTN_EINVAL;
  *BH_out = BH;
  *chunks = 1;
  *chunk_len = N;
  *ws_bytes = 0;
  if (BH == 0 || N == 0 || io_dtype == LIN_ATTN_F32) return LIN_ATTN_OK;
  int cus = 0;
  const int rc = cu_count(&cus);
  if (rc != LIN_ATTN_OK) return rc;
  lal::state_split_plan(BH, N, cus, chunks, chunk_len);
  int64_t groups;
  if (!mul_ok(BH, *chunks, &groups) || groups > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  if (!mul_ok((*chunks - 1) * BH, d * d * 4, ws_bytes)) return LIN_ATTN_EINVAL;
  return LIN_ATTN_OK;
}

}  // namespace

int64_t lin_attn_state_accumulate_split_workspace(int64_t B, int64_t H, int64_t N, int64_t d,
                                                  lin_attn_dtype_t io_dtype) {
  int64_t BH, chunks, chunk_len, ws;
  const int rc = split_check(B, H, N, d, io_dtype, &BH, &chunks, &chunk_len, &ws);
  return rc == LIN_ATTN_OK ? ws : rc;
}

int lin_attn_state_accumulate_split(const void *k, const void *v, float *state, int64_t B, int64_t H, int64_t N,
                                    int64_t d, lin_attn_dtype_t io_dtype, void *workspace, int64_t workspace_bytes,
                                    void *stream) {
  int64_t BH, chunks, chunk_len, ws;
  const int rc = split_check(B, H, N, d, io_dtype, &BH, &chunks, &chunk_len, &ws);
  if (rc != LIN_ATTN_OK) return rc;
  if (workspace_bytes < ws) return LIN_ATTN_EINVAL;
  if (BH == 0 || N == 0) return LIN_ATTN_OK;
  if (io_dtype == LIN_ATTN_F32) return lin_attn_state_accumulate(k, v, state, B, H, N, d, io_dtype, stream);
  if (!ok_ptr(k) || !ok_ptr(v) || !ok_ptr(state)) return LIN_ATTN_EINVAL;
  if (ws > 0 && !ok_ptr(workspace)) return LIN_ATTN_EINVAL;
  lal::StateSplitArgs a{(const unsigned short *)k, (const unsigned short *)v, state, (float *)workspace,
                        N, BH, chunks, chunk_len, 0, nullptr};
  return from_hip(lal::state_split_launch(a, (int)d, (hipStream_t)stream));
}

namespace {

// Prefill cut along the tokens: P parts per sequence (B*H*P at most the
// device's compute units, parts of at least 256 tokens, P a power of two
// dividing N) of L = N/P tokens.
//  - At d = 128, up to kPartMaxOneLaunch parts run in one launch: each part
//    but the last sums its own K^T V and publishes it, and the parts then
//    form every part's start state together, each for 1/P of the elements.
//    Workspace: 2 (P-1) BH states, then three flag arrays of BH P
//    kPartMaxSplit 64-bit words.  (At d = 64 the states are a quarter of the
//    size, the two launches' cached reads of them are cheap, and the
//    exchanges between parts would cost more than the launch they save.)
//  - Otherwise two launches: the K^T V of the first P-1 parts is
//    summed in chunks of L/S tokens (S a power of two <= 4 dividing L, chunks
//    of at least 1024 tokens) by a pass of (P-1) S BH workgroups.
//    Workspace: (P-1) S BH partial states, then a copy of the BH initial
//    states.
struct SeqSplitPlan {
  int64_t BH, P, L, S, ws_bytes;
  bool one_launch;
};

int seqsplit_check(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype,
                   SeqSplitPlan *pl) {
  if (B < 0 || H < 0 || N < 0 || d < 0 || block < 0) return LIN_ATTN_EINVAL;
  if (io_dtype != LIN_ATTN_F32 && io_dtype != LIN_ATTN_BF16) return LIN_ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return LIN_ATTN_EUNSUPPORTED;
  const int max_block = io_dtype == LIN_ATTN_BF16 ? lal::prefill_bf16_max_block((int)d)
                                                  : lal::prefill_f32_max_block((int)d);
  if (block < 16 || block > max_block || block % 16 != 0) return LIN_ATTN_EUNSUPPORTED;
  int64_t BH, total;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &total) || !mul_ok(total, d, &total)) return LIN_ATTN_EINVAL;
  pl->BH = BH;
  pl->P = 1;
  pl->S = 1;
  pl->ws_bytes = 0;
  if (io_dtype == LIN_ATTN_BF16 && BH > 0 && N > 0) {
    int cus = 0;
    const int rc = cu_count(&cus);
    if (rc != LIN_ATTN_OK) return rc;
    while (BH * pl->P * 2 <= cus && N % (pl->P * 2) == 0 && N / (pl->P * 2) >= 256) pl->P *= 2;
  }
  pl->L = pl->P > 0 ? N / pl->P : N;
  pl->one_launch = pl->P > 1 && pl->P <= lal::kPartMaxOneLaunch && d == 128;
  if (pl->one_launch) {
    int64_t states, flags;
    if (!mul_ok(2 * (pl->P - 1) * BH, d * d * 4, &states) || !mul_ok(BH * pl->P, 3 * lal::kPartMaxSplit * 8, &flags))
      return LIN_ATTN_EINVAL;
    pl->ws_bytes = states + flags;
  } else if (pl->P > 1) {
    while (pl->S < 4 && pl->L % (pl->S * 2) == 0 && pl->L / (pl->S * 2) >= 1024) pl->S *= 2;
    const int64_t states = (pl->P - 1) * pl->S * BH + BH;
    if (!mul_ok(states, d * d * 4, &pl->ws_bytes)) return LIN_ATTN_EINVAL;
  }
  return LIN_ATTN_OK;
}

}  // namespace

int64_t lin_attn_prefill_seqsplit_workspace(int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                                            lin_attn_dtype_t io_dtype) {
  SeqSplitPlan pl;
  const int rc = seqsplit_check(B, H, N, d, block, io_dtype, &pl);
  return rc == LIN_ATTN_OK ? pl.ws_bytes : rc;
}

namespace {

// A 64-bit value that differs from call to call (and from what a workspace
// is likely to hold): a random seed plus a call counter, through the
// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014).  Zero is skipped: it is the value
// of a cleared flag.
uint64_t next_part_epoch() {
  static const uint64_t seed = [] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^
           (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  }();
  static std::atomic<uint64_t> calls{0};
  uint64_t z;
  do {
    z = seed + (calls.fetch_add(1, std::memory_order_relaxed) + 1) * 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
  } while (z == 0);
  return z;
}

// Bound of each wait between the parts of a one-launch cut, in ticks of the
// 100 MHz constant clock: about one second, or LIN_ATTN_PART_WAIT_TICKS from
// the environment (a test setting: a small bound makes waits run out and
// their parts' results NaN, which shows that every wait ends).
uint64_t part_wait_ticks() {
  const char *ev = getenv("LIN_ATTN_PART_WAIT_TICKS");
  if (ev && *ev) {
    char *end = nullptr;
    const unsigned long long v = strtoull(ev, &end, 10);
    if (end && *end == 0) return v;
  }
  return lal::kPartWaitTicks;
}

// The launches of a prefill cut along the tokens (plan pl, P > 1), with the
// workspace at `workspace` (pl.ws_bytes bytes).
// One-launch plan: the parts as B*H*P sequences of L tokens, each part but
// the last summing its own K^T V into the workspace first (see
// kPsPartLB).  The flag words are compared with this call's epoch, so their
// contents on entry do not matter unless they hold that random 64-bit value;
// the call leaves the words it used zero.
// Two-launch plan (every workspace byte read is written earlier in the call):
//  1. the K^T V sums of the first P-1 parts, (P-1) S chunks per sequence,
//     into the workspace; the chunk-0 workgroups also copy S_0 there (the
//     state buffer is overwritten by the last part during launch 2, while
//     other parts may still be reading their start);
//  2. the parts as B*H*P sequences of L tokens (contiguous in memory): each
//     forms its initial state from S_0 and the sums of the parts before it,
//     in part order, and the last part of each sequence writes S_N.
int seqsplit_run(const SeqSplitPlan &pl, const void *q, const void *k, const void *v, void *o, float *state,
                 int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype, void *workspace, void *stream) {
  (void)io_dtype;  // bf16: the plan cuts bf16 sequences only
  hipStream_t s = (hipStream_t)stream;
  const int64_t parts = pl.BH * pl.P;
  int cus = 0;
  int rc = cu_count(&cus);
  if (rc != LIN_ATTN_OK) return rc;
  int nsplit = 1;
  while (nsplit < lal::prefill_bf16_max_split((int)d) && parts * nsplit < cus) nsplit *= 2;
  static_assert(lal::kPartMaxSplit >= 4, "flag arrays hold every value slice");
  if (parts * nsplit > 0x7fffffff) return LIN_ATTN_EUNSUPPORTED;
  if (pl.L / block > 0x7ffffff0) return LIN_ATTN_EUNSUPPORTED;
  float *partial = (float *)workspace;
  lal::PrefillArgs a{};
  a.q = (const unsigned short *)q; a.k = (const unsigned short *)k; a.v = (const unsigned short *)v;
  a.o = (unsigned short *)o; a.state = state; a.N = pl.L; a.blk = (int)block; a.nsplit = nsplit;
  a.part_BH = pl.BH; a.part_P = (int)pl.P; a.part_S = 1;
  if (pl.one_launch) {
    a.part_sums = partial;
    a.part_sums_w = partial;
    a.part_flags = (unsigned long long *)(partial + 2 * (size_t)(pl.P - 1) * pl.BH * d * d);
    a.part_epoch = next_part_epoch();
    a.part_wait_ticks = part_wait_ticks();
    return from_hip(lal::prefill_bf16_part_lb_launch(a, parts, (int)d, s));
  }
  float *s0_copy = partial + (size_t)(pl.P - 1) * pl.S * pl.BH * d * d;
  lal::StateSplitArgs sa{(const unsigned short *)k, (const unsigned short *)v, state, partial,
                         N, pl.BH, (pl.P - 1) * pl.S, pl.L / pl.S, 1, s0_copy};
  rc = from_hip(lal::state_split_launch(sa, (int)d, s));
  if (rc != LIN_ATTN_OK) return rc;
  a.part_s0 = s0_copy; a.part_sums = partial; a.part_S = (int)pl.S;
  return from_hip(lal::prefill_bf16_part_launch(a, parts, (int)d, s));
}

}  // namespace

int lin_attn_prefill_seqsplit(const void *q, const void *k, const void *v, void *o, float *state, int64_t B,
                              int64_t H, int64_t N, int64_t d, int64_t block, lin_attn_dtype_t io_dtype,
                              void *workspace, int64_t workspace_bytes, void *stream) {
  SeqSplitPlan pl;
  int rc = seqsplit_check(B, H, N, d, block, io_dtype, &pl);
  if (rc != LIN_ATTN_OK) return rc;
  if (workspace_bytes < pl.ws_bytes) return LIN_ATTN_EINVAL;
  if (pl.P == 1) return prefill_impl(q, k, v, o, state, nullptr, 0, B, H, N, d, block, io_dtype, 0, stream);
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(state) || !ok_ptr(workspace))
    return LIN_ATTN_EINVAL;
  return seqsplit_run(pl, q, k, v, o, state, N, d, block, io_dtype, workspace, stream);
}

int64_t lin_attn_scratch_bytes(void) { return kScratchBytes; }

int lin_attn_prefill_seqsplit_noalloc(const void *q, const void *k, const void *v, void *o, float *state,
                                      int64_t B, int64_t H, int64_t N, int64_t d, int64_t block,
                                      lin_attn_dtype_t io_dtype, void *stream) {
  SeqSplitPlan pl;
  int rc = seqsplit_check(B, H, N, d, block, io_dtype, &pl);
  if (rc != LIN_ATTN_OK) return rc;
  if (pl.ws_bytes > kScratchBytes) return LIN_ATTN_ESCRATCH;
  if (pl.P == 1) return prefill_impl(q, k, v, o, state, nullptr, 0, B, H, N, d, block, io_dtype, 0, stream);
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(state)) return LIN_ATTN_EINVAL;
  void *ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc != LIN_ATTN_OK) return rc;
  return seqsplit_run(pl, q, k, v, o, state, N, d, block, io_dtype, ws, stream);
}

const char *lin_attn_strerror(int code) {
  switch (code) {
    case LIN_ATTN_OK: return "success";
    case LIN_ATTN_EINVAL: return "invalid argument (null or misaligned pointer, negative or overflowing size)";
    case LIN_ATTN_EUNSUPPORTED: return "unsupported configuration (head dim, block size, split or dtype)";
    case LIN_ATTN_EHIP: return "HIP runtime error";
    case LIN_ATTN_ESCRATCH:
      return "the call needs more scratch memory than the library's fixed per-device buffer holds "
             "(lin_attn_scratch_bytes())";
    default: return "unknown error code";
  }
}

}  // extern "C"
