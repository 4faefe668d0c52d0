/*
 * moet_instrument.h - instrumentation hooks of libmoet, kept apart from the
 * layer's ABI (include/moet.h): nothing here changes what any call computes,
 * and a caller that does not time kernels never needs it.
 */
#ifndef MOET_INSTRUMENT_H
#define MOET_INSTRUMENT_H

#include <stddef.h>
#include <stdint.h>

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
int moet_set_timing_events(void *start, void *stop);

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
int moet_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOET_INSTRUMENT_H */
