/* aq_bench.h -- measurement helpers of libaq (gfx950).
 *
 * Not part of the quantized-matmul path: these give the benchmark its second
 * denominators next to the published peaks -- the streaming-read rate this
 * device reaches at a given byte count, and the shader clock and matrix-core
 * rate under a pure MFMA load.  Same conventions as aq.h: device pointers,
 * the caller's stream as void *, nothing allocated, arguments validated on
 * the host before anything is enqueued. */
#ifndef AQ_BENCH_H
#define AQ_BENCH_H

#include <stdint.h>

#include "aq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `buf` once, as a plain streaming
 * kernel: `blocks` workgroups of 256 threads, each thread loading 16 bytes
 * per access, `unroll` (1, 4 or 8) accesses in flight per thread.  Nothing
 * is written except, practically never, one word of `sink` (device), which
 * keeps the loads alive.  buf 16-byte aligned, bytes a multiple of 16;
 * blocks in [1, 65535].  AQ_ERR_INVALID_ARG / AQ_ERR_ALIGNMENT otherwise. */
aq_status aq_bench_stream_read(const void *buf, int64_t bytes, int blocks, int unroll,
                               uint32_t *sink, void *stream);

/* Read `bytes` bytes at `buf` once, in one-shot form: workgroups of `threads`
 * (256, 512 or 1024) threads, each thread issuing all of its `unroll` (4, 8
 * or 16) 16-byte loads before using any; workgroup b reads the contiguous
 * block of threads * unroll * 16 bytes at b times that size.  Same sink,
 * alignment and error conventions as aq_bench_stream_read (AQ_ERR_UNSUPPORTED
 * past 2^31 - 1 workgroups). */
aq_status aq_bench_read_oneshot(const void *buf, int64_t bytes, int threads, int unroll,
                                uint32_t *sink, void *stream);

/* Run `iters` rounds of 14 independent v_mfma_f32_32x32x16_bf16 per wave on
 * `blocks` workgroups of 4 waves (one per SIMD when blocks <= the CU count)
 * and record, per wave, the shader-clock cycles (s_memtime) and the 100 MHz
 * real-time ticks (s_memrealtime) spent in the loop: out[2*w] = cycles,
 * out[2*w + 1] = ticks for wave w = 4*block + wave-in-block (device, uint64
 * [8*blocks]).  cycles / (ticks / 1e8) is the clock under MFMA load;
 * 4*blocks*14*iters*32768 flop / (ticks / 1e8) the MFMA-only rate.
 * blocks in [1, 65535], iters in [1, 1 << 24]. */
aq_status aq_bench_mfma_clock(int blocks, int iters, uint64_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQ_BENCH_H */
