/*
 * stream_probe.h -- C ABI of libstreamprobe, a plain streaming read and a
 * plain copy used as the measured HBM ceilings of the quantile-balancing
 * passes (a diagnostic library, separate from libqb; the method never
 * calls it).
 *
 * Both passes of the exact quantile balancing update ("Exact Quantile
 * Balancing and Load-Error Injection for Mixture-of-Experts", summary page,
 * EQB paragraph: the margins are streamed once per byte pass) are bounded
 * by how fast one GPU can stream the score matrix; this kernel streams a
 * buffer with no other work, so its rate is that bound as measured.
 *
 *   sp_read:  loads every byte of p[0, bytes) once; an integer fold of the
 *             data is kept live and written to sink[blockIdx] only on a value the
 *             data practically never produces (no write traffic).
 *   sp_read_nt: sp_read with non-temporal loads (the streaming hint): on
 *             MI355X the faster way to read a buffer once, as the passes do
 *             for layers far larger than the Infinity Cache.
 *   sp_copy:  loads every byte of src[0, bytes) once and stores it to the
 *             same offset of dst (a plain copy: the ceiling of the passes that
 *             read and write equal amounts, such as the LEI gradient offsets
 *             of the same page's LEI paragraph); src and dst must not overlap;
 *             unroll 1, 2, 4 or 8.
 *   p, src, dst: DEVICE pointers, 16-byte aligned, caller-owned; bytes a positive
 *   multiple of 16.  sink: device
 *   uint32 [grid].  grid: workgroups of 1024 threads (1 .. 2^20); unroll:
 *   16-byte loads in flight per thread (1, 2, 4, 8 or 16).  Asynchronous on
 *   `stream` (a hipStream_t; NULL = null stream); nothing is allocated.
 *   Returns SP_OK, SP_EINVAL (bad pointer, size, alignment, grid or unroll;
 *   nothing launched) or SP_EHIP (the launch failed).
 */
#ifndef STREAM_PROBE_H
#define STREAM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SP_API __attribute__((visibility("default")))

typedef struct ihipStream_t* sp_stream_t; /* same type as hipStream_t */

enum { SP_OK = 0, SP_EINVAL = -1, SP_EHIP = -3 };

SP_API int sp_read(const void* p, int64_t bytes, int grid, int unroll, uint32_t* sink, sp_stream_t stream);
SP_API int sp_read_nt(const void* p, int64_t bytes, int grid, int unroll, uint32_t* sink, sp_stream_t stream);
SP_API int sp_copy(const void* src, void* dst, int64_t bytes, int grid, int unroll, sp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_PROBE_H */
