/*
 * moet_instrument.h - instrumentation hooks of libmoet, kept apart from the
 * layer's ABI (include/moet.h): nothing here changes what any call computes,
 * and a caller that does not time kernels never needs it.
 */
#ifndef MOET_INSTRUMENT_H
#define MOET_INSTRUMENT_H

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

#ifdef __cplusplus
}
#endif

#endif /* MOET_INSTRUMENT_H */
