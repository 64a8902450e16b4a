/*
 * Measurement helper for the benchmark (libfi_bench.so, not part of the
 * attention library's interface).
 *
 * fi_bench_stream_read: reads `bytes` bytes at `buf` (device memory, 16-byte
 * aligned, a multiple of 16 bytes) once with 16-byte nontemporal loads from
 * 1024 work-groups of 256 threads, asynchronously on `stream` (a
 * hipStream_t, or NULL for the null stream). The loaded words are folded so
 * no load can be elided; `sink` (device, 4 bytes) is written only if the
 * fold hits one fixed constant. Over a buffer much larger than the caches,
 * bytes / duration is the practical HBM read ceiling a bandwidth-bound kernel
 * compares itself with. Returns 0 (hipSuccess) or the hipError_t of a
 * refused argument or failed launch. Nothing is allocated; the caller owns
 * both buffers.
 */
#ifndef FI_BENCH_H_
#define FI_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int fi_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FI_BENCH_H_ */
