/*
 * la2_test_hooks.h -- plan overrides and a measurement stream of the test build
 * of the library.
 *
 * Only lib/libla2_testhooks.so (the same sources compiled with LA2_TEST_HOOKS,
 * plus la2_stream.hip) exports these functions; the release library
 * lib/libla2.so does not, and its launch plan depends on the call's arguments
 * alone.  The tests use it to
 * force work decompositions that the automatic plan would not pick for small
 * shapes, so that those code paths are checked against the oracle.
 *
 * la2_test_set_plan sets process-wide state read by every later call of that
 * library: not thread-safe, and meant for single-threaded test processes only.
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
 *   legacy_forward: non-zero runs the forward-direction bf16 output scans at d = d_v = 128
 *                  on the eight-wave scan kernel instead of the producer/consumer one,
 *                  and la2_forward_normalized there as its denominator pass and numerator scan
 *                  instead of the one fused launch
 *   legacy_dkdv:   non-zero runs the fused dK/dV pass at d = d_v = 128 on its eight-wave kernel instead
 *                  of the producer/consumer walk of the one-pass backward
 *   reverse_prefix: non-zero launches the reverse segment prefix even where the backward walk would
 *                  sum the state deltas of its (at most two) later pieces itself
 * Returns LA2_OK. */
int la2_test_set_plan(int64_t seg_tiles, int state_sub, int slice_width, int separate_dkdv,
                      int64_t norm_segment, int two_pass_backward, int legacy_forward, int legacy_dkdv,
                      int reverse_prefix);

/* A plain HBM stream, for measuring what the tile kernels' read:write mixes can reach:
 * dst_j = src_0 + ... + src_{nsrc-1} (u32 lanes) over `bytes` bytes of each device buffer, read and
 * written as 16-byte lane accesses by a grid-stride loop of `blocks` workgroups of `threads`
 * threads, with the nontemporal cache hint when `nontemporal` is non-zero; enqueued on `stream`.
 *   src: nsrc (1-4) device pointers; dst: ndst (1-3) device pointers; all 16-byte aligned,
 *   bytes a multiple of 16; threads a multiple of 64 in [64, 1024].
 * Returns LA2_OK, LA2_ERR_BAD_SHAPE, LA2_ERR_NULL_POINTER (a NULL or misaligned pointer) or
 * LA2_ERR_HIP. */
int la2_test_stream(const void *const *src, int nsrc, void *const *dst, int ndst, size_t bytes,
                    int blocks, int threads, int nontemporal, void *stream);

/* Enqueue on `stream` a probe of the memory-side cache (test build only): device buffers q, k, v, o of
 * `bytes` each are cut into items of `item_bytes`, one workgroup of 512 threads (144 KiB of LDS, one
 * per CU) per item.  Phase A reads the item's k and v; phase B reads its q, k, v and writes its o.
 * mode 0: B alone; 1: A then B in the same workgroup (A's loads with the default cache policy, so B's
 * second read of k and v may come from the cache); 2: A alone (writes one 16-byte chunk per item
 * into o).  nontemporal sets the hint on B's accesses (and on A's in mode 2).  The time of mode 1
 * against modes 0 and 2 shows what a state-only pass fused ahead of the output pass would cost at
 * that item size.  bytes a multiple of item_bytes (at most 2^31 - 1 items), item_bytes a multiple
 * of 16, pointers 16-byte aligned.  Returns LA2_OK, LA2_ERR_BAD_SHAPE, LA2_ERR_NULL_POINTER or
 * LA2_ERR_HIP. */
int la2_test_reread(const void *q, const void *k, const void *v, void *o, size_t bytes, size_t item_bytes,
                    int mode, int nontemporal, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LA2_TEST_HOOKS_H */
