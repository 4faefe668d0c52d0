/*
 * moet_instrument.h - instrumentation hooks of libmoet, kept apart from the
 * layer's ABI (include/moet.h): nothing here changes what any call computes,
 * and a caller that does not time kernels never needs it.
 */
#ifndef MOET_INSTRUMENT_H
#define MOET_INSTRUMENT_H

#include <stddef.h>
#include <stdint.h>

#include "moet.h"   /* moet_status */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moet_set_timing_events - benchmark instrumentation.  While set (per host
 * thread), every moet_moe_forward call launches its first expert kernel (the
 * gate/up kernel) with hipExtLaunchKernel and these two events, which the
 * runtime stamps at that kernel's start and end (no marker packets between
 * the launches), so the caller can time that one kernel with
 * hipEventElapsedTime.  `start` / `stop` are caller-owned hipEvent_t handles;
 * pass NULL, NULL to disable.  Returns MOET_EINVAL if only one is NULL.
 */
moet_status moet_set_timing_events(void *start, void *stop);

/* Words of the sink array moet_probe_read writes. */
#define MOET_PROBE_SINK_WORDS 8192

/*
 * moet_probe_read - measurement reference: reads every byte of `src` once
 * with 16-byte loads in a grid-stride loop over 1024 workgroups of 4 waves
 * (the fastest streaming-read shape measured on MI355X), and writes one xor
 * word per wave to `sink` (uint32 [MOET_PROBE_SINK_WORDS], device) so that
 * no load can be dropped.  Timing it gives the achievable HBM read rate
 * on the running device; it also evicts the caches without dirtying them.
 * src: device memory, `bytes` long (a positive multiple of 16).  Enqueued on
 * `stream`.  Returns MOET_EINVAL for NULL or misaligned pointers or a bad
 * size, MOET_EHIP if the launch fails.
 */
moet_status moet_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

enum { MOET_PROBE_MFMA_BF16 = 0, MOET_PROBE_DOT2_BF16 = 1 };

/*
 * moet_probe_peak - measurement reference: the sustained issue rate of one
 * instruction with no memory traffic, over 1024 workgroups of 4 waves (4 per
 * CU).  Each wave runs `iters` rounds of 4 (MFMA) or 8 (dot2) independent
 * accumulation chains and writes one word to `sink` (uint32
 * [MOET_PROBE_SINK_WORDS], device) so that nothing can be dropped.
 *   MOET_PROBE_MFMA_BF16: v_mfma_f32_32x32x16_bf16, 32,768 flops each, 4 per
 *     round per wave: flops = 1024 * 4 * 4 * iters * 32768.
 *   MOET_PROBE_DOT2_BF16: v_dot2_f32_bf16, 8 per round per wave:
 *     wave instructions = 1024 * 4 * 8 * iters.
 * Timing it gives the matrix-core and vector-ALU peaks the running device
 * sustains (its clock under that load included).  Returns MOET_EINVAL for a
 * NULL or misaligned sink, iters < 1 or an unknown kind, MOET_EHIP if the
 * launch fails.
 */
moet_status moet_probe_peak(int kind, int32_t iters, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOET_INSTRUMENT_H */
