/*
 * q4_measure.h -- measurement kernels of the gfx950 library: the floors that
 * the decode kernels are compared against on the running GPU.
 *
 * The benchmark states the decode GEMV's weight bandwidth both against the
 * published HBM peak and against what this GPU measurably does for the same
 * bytes: meTile PR #29 ("Why int4 wins is bandwidth, not batching") reports
 * effective bandwidth against a measured streaming ceiling. Two floors:
 *   - an empty kernel: the cost of one dispatch of a given launch shape,
 *     back to back on one stream;
 *   - a read-only stream: every byte of a buffer read once with 128-bit
 *     non-temporal loads, nothing written but one word. A read of the decode
 *     step's weight bytes is the fastest any kernel can take them in.
 * These kernels are not on the product path; they share the library so that
 * one build serves both.
 *
 * Arguments: grid, block > 0 with block a multiple of 64 and at most 1024.
 * buf: device pointer, 16-byte aligned, bytes a multiple of 16 below 2^31.
 * sink: device pointer to one uint32, written only if the XOR of every dword
 * read equals `key` (pass a value the data does not produce; the write keeps
 * the loads from being removed). Returns a q4_status (q4.h); nothing is
 * launched on an invalid call.
 */
#ifndef Q4_MEASURE_H
#define Q4_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int q4_measure_empty(int grid, int block, void* stream);
int q4_measure_stream_read(const void* buf, size_t bytes, int grid, int block, uint32_t key, uint32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_MEASURE_H */
