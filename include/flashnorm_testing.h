/*
 * flashnorm_testing.h -- a test-only switch of libflashnorm.so.  Nothing
 * here is part of the method; a program that computes with the library
 * never calls it.
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

#ifdef __cplusplus
}
#endif

#endif /* FLASHNORM_TESTING_H */
