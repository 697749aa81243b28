/*
 * kvbt_bench.h -- measurement helpers exported by libkvbt.so. They are not part of
 * the selector; the benchmark uses them to put the selector's timings in context:
 * the launch floor of an empty kernel, the bandwidth and HBM counter readings of a
 * plain device-to-device copy of known size, and the bandwidth of a read-only stream
 * in the long-row selector's access pattern (the achievable read ceiling).
 *
 * Pointers are device pointers; `stream` is a hipStream_t (NULL = default stream).
 * All calls are asynchronous and return 0, KVBT_E_NULL / KVBT_E_RANGE for bad
 * arguments (nothing launched), or KVBT_E_LAUNCH.
 */
#ifndef KVBT_BENCH_H
#define KVBT_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch one empty kernel of `blocks` workgroups of 64 threads (1 <= blocks <= 2^20). */
int kvbt_bench_empty(int blocks, void* stream);

/* Copy `bytes` (a positive multiple of 16; both pointers 16-byte aligned) from src to
 * dst with a grid-stride kernel of 16-byte loads and stores. */
int kvbt_bench_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* Read `bytes` (a positive multiple of 16; src 16-byte aligned) once: one wavefront per
 * 32 KiB segment, 16-byte nontemporal loads, two 4 KiB chunks in flight. `sink` must
 * point to at least 4 writable device bytes; it is written only for one checksum value
 * that the data never produces in practice. */
int kvbt_bench_read(const void* src, int64_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVBT_BENCH_H */
