// Streaming kernels that measure the HBM bandwidth a plain, well-coalesced
// kernel reaches for a given read:write byte mix (a reference rate for the
// attention kernels' own mixes; not a bound on them).  It is measurement
// infrastructure, not part of the attention library: bench.py loads it (as
// _lib/libhbm_stream.so) to put the attention kernels' rates beside the
// practical ceiling of their own traffic mix (the prefill reads three bytes
// per byte it writes, the decode step one).
//
// Work is cut into units of 256 lanes x 16 bytes.  A unit reads RD such
// slices (16-byte non-temporal loads, consecutive lanes at consecutive
// addresses) and, when writes are on, writes one slice of their XOR.  Each
// workgroup takes a contiguous run of units and walks it BATCH units at a
// time: all loads of a batch are issued before its stores, so a wave keeps
// BATCH * RD loads in flight.  With one read per write, source and
// destination may be the same buffer: each lane then writes its slice back
// to the address it read (a read-modify-write stream).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hbm_stream.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT_STORE>
__device__ __forceinline__ void put(u32x4 *p, u32x4 x) {
  if constexpr (NT_STORE)
    __builtin_nontemporal_store(x, p);
  else
    *p = x;
}

// `salt` is zero at run time.  Writing back the loaded value unchanged would
// let the compiler drop an in-place stream's stores and loads.
template <int RD, bool WRITE, bool NT_STORE, int BATCH>
__device__ __forceinline__ void stream_run(const u32x4 *src, u32x4 *dst, int64_t units, int64_t per_wg,
                                           unsigned salt) {
  const int64_t u0 = (int64_t)blockIdx.x * per_wg;
  const int64_t u1 = u0 + per_wg < units ? u0 + per_wg : units;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t u = u0;
  for (; u + BATCH <= u1; u += BATCH) {
    u32x4 x[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const u32x4 *s = src + (u + b) * RD * 256 + threadIdx.x;
      x[b] = u32x4{salt, salt, salt, salt};
#pragma unroll
      for (int r = 0; r < RD; ++r) x[b] ^= __builtin_nontemporal_load(s + r * 256);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if constexpr (WRITE)
        put<NT_STORE>(dst + (u + b) * 256 + threadIdx.x, x[b]);
      else
        acc ^= x[b];
    }
  }
  for (; u < u1; ++u) {  // the run's last units, fewer than a batch
    const u32x4 *s = src + u * RD * 256 + threadIdx.x;
    u32x4 x = {salt, salt, salt, salt};
#pragma unroll
    for (int r = 0; r < RD; ++r) x ^= __builtin_nontemporal_load(s + r * 256);
    if constexpr (WRITE)
      put<NT_STORE>(dst + u * 256 + threadIdx.x, x);
    else
      acc ^= x;
  }
  // read-only runs keep their loads alive through a store that never happens
  // for the fill patterns used (all bytes equal give acc[0] == acc[1])
  if constexpr (!WRITE)
    if (acc[0] != acc[1]) dst[threadIdx.x] = acc;
}

template <int RD, bool WRITE, bool NT_STORE, int BATCH>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                      int64_t units, int64_t per_wg, unsigned salt) {
  stream_run<RD, WRITE, NT_STORE, BATCH>(src, dst, units, per_wg, salt);
}

// the in-place stream: one pointer, no aliasing promise
template <bool NT_STORE, int BATCH>
__global__ __launch_bounds__(256) void in_place_kernel(u32x4 *buf, int64_t units, int64_t per_wg,
                                                       unsigned salt) {
  stream_run<1, true, NT_STORE, BATCH>(buf, buf, units, per_wg, salt);
}

template <int RD, bool WRITE, bool NT, int BATCH>
void launch(const void *src, void *dst, int64_t units, int wgs, hipStream_t stream) {
  const int64_t per = (units + wgs - 1) / wgs;
  if (src == dst)
    in_place_kernel<NT, BATCH><<<wgs, 256, 0, stream>>>((u32x4 *)dst, units, per, 0u);
  else
    stream_kernel<RD, WRITE, NT, BATCH><<<wgs, 256, 0, stream>>>((const u32x4 *)src, (u32x4 *)dst, units, per, 0u);
}

template <int BATCH>
int dispatch(const void *src, void *dst, int64_t units, int rd, int write, int nt, int wgs, hipStream_t stream) {
  if (rd == 1 && write)
    nt ? launch<1, true, true, BATCH>(src, dst, units, wgs, stream)
       : launch<1, true, false, BATCH>(src, dst, units, wgs, stream);
  else if (rd == 3 && write)
    nt ? launch<3, true, true, BATCH>(src, dst, units, wgs, stream)
       : launch<3, true, false, BATCH>(src, dst, units, wgs, stream);
  else if (rd == 1 && !write)
    launch<1, false, false, BATCH>(src, dst, units, wgs, stream);
  else
    return -2;
  return 0;
}

// Role-split stream, the traffic shape of the prefill (one workgroup per
// compute unit streaming three inputs in and one output out): in each
// workgroup of 4 waves, wave w < 3 reads units [u0, u1) of the w-th third of
// src (DEPTH 16-byte loads per lane in flight) and wave 3 writes units
// [u0, u1) of dst with a fixed pattern.  The reads feed a store that equal
// bytes never take, so they cannot be dropped.
template <int DEPTH, bool NT_STORE>
__global__ __launch_bounds__(256) void roles_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                     int64_t units, int64_t per_wg, unsigned salt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t u0 = (int64_t)blockIdx.x * per_wg;
  const int64_t u1 = u0 + per_wg < units ? u0 + per_wg : units;
  if (u0 >= u1) return;
  const int64_t n = (u1 - u0) * 256;  // 16-byte pieces of the run
  if (wave < 3) {
    const u32x4 *s = src + ((int64_t)wave * units + u0) * 256 + lane;
    u32x4 acc = {salt, salt, salt, salt};
    int64_t i = 0;
    for (; i + 64 * DEPTH <= n; i += 64 * DEPTH) {
      u32x4 x[DEPTH];
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) x[b] = __builtin_nontemporal_load(s + i + 64 * b);
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) acc ^= x[b];
    }
    for (; i < n; i += 64) acc ^= __builtin_nontemporal_load(s + i);
    if (acc[0] != acc[1]) dst[lane] = acc;
  } else {
    u32x4 *d = dst + u0 * 256 + lane;
    const u32x4 v = {salt ^ 0x9e3779b9u, salt ^ 0x7f4a7c15u, salt ^ 0x94d049bbu, salt ^ 0x2545f491u};
    for (int64_t i = 0; i < n; i += 64) put<NT_STORE>(d + i, v);
  }
}

template <int DEPTH>
void launch_roles(const void *src, void *dst, int64_t units, int nt, int wgs, hipStream_t stream) {
  const int64_t per = (units + wgs - 1) / wgs;
  if (nt)
    roles_kernel<DEPTH, true><<<wgs, 256, 0, stream>>>((const u32x4 *)src, (u32x4 *)dst, units, per, 0u);
  else
    roles_kernel<DEPTH, false><<<wgs, 256, 0, stream>>>((const u32x4 *)src, (u32x4 *)dst, units, per, 0u);
}

}  // namespace

extern "C" int hbm_stream_roles(const void *src, void *dst, int64_t units, int nt_store, int workgroups, int depth,
                                hipStream_t stream) {
  if (!src || !dst || units < 0 || workgroups <= 0 || src == dst) return -1;
  if (depth != 4 && depth != 8 && depth != 16) return -2;
  if (units == 0) return 0;
  if (depth == 4) launch_roles<4>(src, dst, units, nt_store, workgroups, stream);
  else if (depth == 8) launch_roles<8>(src, dst, units, nt_store, workgroups, stream);
  else launch_roles<16>(src, dst, units, nt_store, workgroups, stream);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hbm_stream(const void *src, void *dst, int64_t units, int reads_per_write, int write,
                          int nt_store, int workgroups, int batch, hipStream_t stream) {
  if (!src || !dst || units < 0 || workgroups <= 0) return -1;
  if (batch != 1 && batch != 4 && batch != 16) return -2;
  if (src == dst && !(reads_per_write == 1 && write)) return -2;
  if (reads_per_write != 1 && !(reads_per_write == 3 && write)) return -2;
  if (units == 0) return 0;
  const int rc =
      batch == 1   ? dispatch<1>(src, dst, units, reads_per_write, write, nt_store, workgroups, stream)
      : batch == 4 ? dispatch<4>(src, dst, units, reads_per_write, write, nt_store, workgroups, stream)
                   : dispatch<16>(src, dst, units, reads_per_write, write, nt_store, workgroups, stream);
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
