/* Streaming bandwidth probes (measurement only; not part of the attention
 * library, built separately as libhbm_stream.so): reference rates for a
 * read:write mix, not bounds on the attention kernels.
 *
 * hbm_stream: one launch of a plain streaming kernel on `stream`.
 *   src, dst      device pointers, 16-byte aligned, owned by the caller; with
 *                 one read per write they may be equal (an in-place stream).
 *   units         work units of 4096 bytes per read slice: the kernel reads
 *                 units * reads_per_write * 4096 bytes of src and, when
 *                 `write` is non-zero, writes units * 4096 bytes of dst
 *                 (src must hold the former, dst the latter; a read-only run
 *                 may store 4096 bytes to dst).
 *   reads_per_write  1 or 3 with writes, 1 without.
 *   nt_store      non-zero: non-temporal stores.
 *   workgroups    workgroups of 256 lanes, each taking a contiguous run of units.
 *   batch         1, 4 or 16: units each wave loads before it stores them.
 * Returns 0, -1 for a null pointer or a bad size, -2 for an unsupported
 * combination, -3 for a launch error.
 */
#ifndef HBM_STREAM_H
#define HBM_STREAM_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int hbm_stream(const void *src, void *dst, int64_t units, int reads_per_write, int write, int nt_store,
               int workgroups, int batch, hipStream_t stream);
/* hbm_stream_roles: the prefill's traffic shape.  Each workgroup of 4 waves
 * takes a contiguous run of `units` (ceil(units / workgroups) each): waves
 * 0..2 read that run of the first, second and third third of src (src holds
 * 3 * units * 4096 bytes), `depth` 16-byte loads per lane in flight (4, 8 or
 * 16), and wave 3 writes that run of dst (units * 4096 bytes) with a fixed
 * pattern.  src and dst must differ.  Same return codes as hbm_stream.
 */
int hbm_stream_roles(const void *src, void *dst, int64_t units, int nt_store, int workgroups, int depth,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
