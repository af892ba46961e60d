/*
 * A measurement probe, not part of the attention path: a plain streaming
 * read of a device buffer, so that the bandwidth the split-KV decode reaches
 * can be set beside what a bare read reaches on the same GPU. Built as its
 * own library, libsattn_probe.so, and used only by `bench.py --read-ceiling`.
 */
#ifndef SATTN_PROBE_H
#define SATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads every byte of `buf` (device memory, `bytes` > 0 and a multiple of
 * 16, 16-byte aligned) once, with 16-byte nontemporal loads: `grid`
 * workgroups of 256 threads, each streaming one contiguous slice, and
 * writes one 32-bit XOR of what each thread read to `out[blockIdx.x * 256 +
 * threadIdx.x]` (device memory of `out_count` >= grid * 256 entries, which
 * keeps the loads from being dropped). Enqueued on `stream` (a hipStream_t,
 * NULL for the default stream); nothing is allocated.
 * Returns 0, or -1 for invalid arguments (nothing enqueued), or -2 if the
 * launch failed.
 */
int sattn_probe_read(const void* buf, int64_t bytes, uint32_t* out, int64_t out_count, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif
