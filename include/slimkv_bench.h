/*
 * slimkv_bench.h -- measurement helpers exported by libslimkv.so beside the
 * attention entry points (include/slimkv.h).  They compute nothing of the
 * attention; they exist so that a benchmark can put the attention kernels'
 * bandwidth next to what a plain kernel reaches on the same device, and can
 * start a timed call with cold caches.
 *
 * The roofline the decode path is judged against is HBM bandwidth: page "Can
 * SlimKV compress KV cache jointly across tokens and features", section
 * "Why feature compression stalls at key reconstruction", names memory
 * access to the KV cache as what limits long-context serving, and the
 * latent path streams every cache byte once per call.
 *
 * Rules as in slimkv.h: device pointers, caller-owned buffers, asynchronous
 * on `stream` (a hipStream_t; NULL is the null stream), every check before
 * any HIP call, a status returned and nothing launched on error.
 */
#ifndef SLIMKV_BENCH_H
#define SLIMKV_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "slimkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * slimkv_bench_stream_read -- the streaming-read ceiling: one kernel that
 * reads `bytes` bytes at `src` once, as 16-byte non-temporal buffer loads
 * (the load the attention kernels use for cache rows), with `in_flight`
 * 16-byte loads outstanding per lane (1 .. 16), over `workgroups` workgroups
 * of 256 threads (0: two per compute unit, the attention kernels' grid), and
 * writes a 32-bit checksum of what it read to sink[0] (so the loads cannot
 * be dropped).  Its time is the fastest a single launch can stream that
 * many bytes on this device; an attention call that moves the same bytes
 * can be compared with it directly.
 *
 *   src   device, 16-byte aligned; `bytes` a multiple of 16 in [16, 2^31 - 16]
 *   sink  device, 4 bytes, written (must not overlap src)
 */
slimkv_status slimkv_bench_stream_read(const void* src, size_t bytes, int32_t in_flight,
                                       int32_t workgroups, uint32_t* sink, void* stream);

/*
 * slimkv_bench_flush -- writes `bytes` bytes of `buf` (16-byte aligned, a
 * multiple of 16) with a pattern derived from `seed`, so that a following
 * timed call finds none of its inputs in the L2 caches or the last-level
 * (MALL) cache: pass a buffer larger than the MALL (256 MB on MI355X; 512 MB
 * or more is the safe size).  Writes only through vector stores.
 */
slimkv_status slimkv_bench_flush(void* buf, size_t bytes, uint32_t seed, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SLIMKV_BENCH_H */
