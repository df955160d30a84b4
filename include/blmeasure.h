/*
 * blmeasure.h -- measurement kernels of the benchmark (libblmeasure.so).
 *
 * Not part of the BitLinear path: reference kernels that the benchmark times
 * beside it, on the same GPU, to state what the memory system delivers.
 * Pointers are DEVICE pointers owned by the caller; the calls only enqueue
 * work on `stream` (a hipStream_t, NULL for the null stream).  Return 0 on
 * success, 1 for bad arguments (nothing enqueued), 2 if the launch failed.
 */
#ifndef BLMEASURE_H
#define BLMEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at `buf` once, as a decode kernel reads packed weights:
 * 16-byte loads marked non-temporal, a wave's load covering 1 KiB
 * contiguously, eight loads per lane in flight, each workgroup sweeping its
 * own contiguous span.  The loaded words are folded (XOR) into one word per
 * workgroup, written to sink[blockIdx] so that the loads cannot be dropped.
 *   buf    16-byte aligned; bytes a positive multiple of 32768.
 *   sink   blmeasure_stream_read_sink_words(bytes) words (written).  */
size_t blmeasure_stream_read_sink_words(size_t bytes);
int blmeasure_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BLMEASURE_H */
