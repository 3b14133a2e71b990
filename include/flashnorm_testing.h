/*
 * flashnorm_testing.h -- test and measurement hooks of libflashnorm.so.
 * Nothing here is part of the method; a program that computes with the
 * library never calls them.
 *
 * The two-stream variant (FN_TWO_STREAM) computes the product on
 * stream_aux and the row scale on stream, then makes stream wait for an
 * event recorded after the product before the post-scale reads it.  The
 * FlashNorm talk write-up (its bullets on the bug and on its root cause and
 * fix) describes what happens without that wait: the post-scale reads a
 * product that is stale or half written, and the outputs lag one step
 * behind their inputs.  A test of the join must be able to see that
 * failure, so this switch removes the join to show that the test catches
 * it.  The reads it causes stay inside the workspace: a data race, never an
 * out-of-bounds access.
 */
#ifndef FLASHNORM_TESTING_H
#define FLASHNORM_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/* skip != 0: later FN_TWO_STREAM calls made by the calling thread skip the
 * wait for the product (the post-scale may read a stale workspace); skip == 0
 * restores the join, the default.  The setting is per host thread.  Returns
 * the previous setting (0 or 1).  Never fails. */
int fn_testing_skip_join(int skip);

/* Timing of the prefill GEMM for a measurement harness (the roofline of a
 * step that launches a pass before or after its GEMM needs the GEMM's own
 * duration).  With n > 0, each later bf16 or fp8 prefill GEMM launch made
 * by the calling thread is bracketed by hipEventRecord(starts[i % n]) and
 * hipEventRecord(stops[i % n]) on the launch stream, i = 0, 1, ... counted
 * from this call; n <= 0 turns the hook off (the default; starts / stops
 * may then be NULL).  starts and stops hold n hipEvent_t handles that the
 * caller created and owns, and both arrays must stay valid while the hook
 * is on; the library only records the events.  Decode kernels (M <= 16)
 * are not bracketed.  The setting is per host thread.
 * Returns 0 (FN_OK), or 1 (FN_E_NULL) when n > 0 and an array is NULL (the
 * hook is then off). */
int fn_testing_gemm_events(void* const* starts, void* const* stops, int n);

#ifdef __cplusplus
}
#endif

#endif /* FLASHNORM_TESTING_H */
