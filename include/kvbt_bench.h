/*
 * kvbt_bench.h -- measurement helpers exported by libkvbt.so. They are not part of
 * the selector; the benchmark uses them to put the selector's timings in context:
 * the launch floor of an empty kernel, and the bandwidth and HBM counter readings
 * of a plain device-to-device copy of known size.
 *
 * Pointers are device pointers; `stream` is a hipStream_t (NULL = default stream).
 * Both calls are asynchronous and return 0, KVBT_E_NULL / KVBT_E_RANGE for bad
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

#ifdef __cplusplus
}
#endif

#endif /* KVBT_BENCH_H */
