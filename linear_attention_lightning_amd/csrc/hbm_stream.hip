// Streaming kernel that measures the HBM bandwidth a plain, well-coalesced
// kernel reaches for a given read:write byte mix.  It is measurement
// infrastructure, not part of the attention library: bench.py loads it (as
// _lib/libhbm_stream.so) to put the attention kernels' rates beside the
// practical ceiling of their own traffic mix (the prefill reads three bytes
// per byte it writes, the decode step one).
//
// Work is cut into units of 256 lanes x 16 bytes.  A unit reads RD such
// slices (16-byte non-temporal loads, consecutive lanes at consecutive
// addresses) and, when RD > 0 and writes are on, writes one slice of their
// XOR.  Each workgroup takes a contiguous run of units.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hbm_stream.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int RD, bool WRITE, bool NT_STORE>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                      int64_t units, int64_t per_wg) {
  const int64_t u0 = (int64_t)blockIdx.x * per_wg;
  const int64_t u1 = u0 + per_wg < units ? u0 + per_wg : units;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t u = u0; u < u1; ++u) {
    const u32x4 *s = src + u * RD * 256 + threadIdx.x;
    u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RD; ++r) x ^= __builtin_nontemporal_load(s + r * 256);
    if constexpr (WRITE) {
      if constexpr (NT_STORE)
        __builtin_nontemporal_store(x, dst + u * 256 + threadIdx.x);
      else
        dst[u * 256 + threadIdx.x] = x;
    } else {
      acc ^= x;
    }
  }
  // read-only runs keep their loads alive through a store that never happens
  // for the fill patterns used (all bytes equal give acc[0] == acc[1])
  if constexpr (!WRITE)
    if (acc[0] != acc[1]) dst[threadIdx.x] = acc;
}

template <int RD, bool WRITE, bool NT>
void launch(const void *src, void *dst, int64_t units, int wgs, hipStream_t stream) {
  const int64_t per = (units + wgs - 1) / wgs;
  stream_kernel<RD, WRITE, NT><<<wgs, 256, 0, stream>>>((const u32x4 *)src, (u32x4 *)dst, units, per);
}

}  // namespace

extern "C" int hbm_stream(const void *src, void *dst, int64_t units, int reads_per_write, int write,
                          int nt_store, int workgroups, hipStream_t stream) {
  if (!src || !dst || units < 0 || workgroups <= 0) return -1;
  if (units == 0) return 0;
  if (reads_per_write == 1 && write)
    nt_store ? launch<1, true, true>(src, dst, units, workgroups, stream)
             : launch<1, true, false>(src, dst, units, workgroups, stream);
  else if (reads_per_write == 3 && write)
    nt_store ? launch<3, true, true>(src, dst, units, workgroups, stream)
             : launch<3, true, false>(src, dst, units, workgroups, stream);
  else if (reads_per_write == 1 && !write)
    launch<1, false, false>(src, dst, units, workgroups, stream);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
