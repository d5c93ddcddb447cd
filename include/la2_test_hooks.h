/*
 * la2_test_hooks.h -- plan overrides of the test build of the library.
 *
 * Only lib/libla2_testhooks.so (the same sources compiled with LA2_TEST_HOOKS)
 * exports this function; the release library lib/libla2.so does not, and its
 * launch plan depends on the call's arguments alone.  The tests use it to
 * force work decompositions that the automatic plan would not pick for small
 * shapes, so that those code paths are checked against the oracle.
 *
 * It sets process-wide state read by every later call of that library: not
 * thread-safe, and meant for single-threaded test processes only.
 */
#ifndef LA2_TEST_HOOKS_H
#define LA2_TEST_HOOKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Force plan choices; 0 leaves a choice automatic (the release plan).
 *   seg_tiles:     tiles per segment of every chain (split chains even when they fill the GPU)
 *   state_sub:     pieces per segment in the state-only pass (when it divides the segment)
 *   slice_width:   64 runs 128-wide bf16 values as two 64-wide slices
 *   separate_dkdv: non-zero computes dk and dv by two separate reverse scans
 *   norm_segment:  positions per segment of the normalized form's denominator scans
 *   two_pass_backward: non-zero runs la2_backward_saved without decay (bf16, d = d_v = 128) as a dQ
 *                  pass and a dK/dV pass instead of the one-pass backward
 * Returns LA2_OK. */
int la2_test_set_plan(int64_t seg_tiles, int state_sub, int slice_width, int separate_dkdv,
                      int64_t norm_segment, int two_pass_backward);

#ifdef __cplusplus
}
#endif

#endif /* LA2_TEST_HOOKS_H */
