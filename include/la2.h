/*
 * la2.h -- C ABI of the MI355X (gfx950) Lightning Attention-2 library.
 *
 * Operation.  Causal linear attention with identity feature map, no
 * denominator and an optional per-head decay lam_h in (0, 1]:
 *
 *     S_t = lam_h * S_{t-1} + k_t v_t^T,     o_t = S_t^T q_t,
 *
 * i.e. the numerator recurrence of page "Lightning Attention"
 * (lizeman.github.io llm-arch-kb), section 1, computed the way its section 2
 * derives: the sequence is cut into tiles of `block` positions; inside a tile
 * the output is the masked left product (Q_b K_b^T (.) M) V_b (Step 2), across
 * tiles the right product Q_b S_{b-1} (Step 3), and the d x d_v state is
 * carried from tile to tile (Step 4).  With lam < 1 the mask M becomes
 * lam^(i-j) on and below the diagonal, the inter-tile rows are weighted
 * lam^(i+1) and the state update is S_b = lam^block S_{b-1} +
 * (diag(lam^(block-1-j)) K_b)^T V_b.  The backward pass is tiled as well
 * (Lightning Attention-2 abstract, arXiv 2401.04658 card): dQ by the same
 * forward-order scan and dK, dV by the mirrored reverse-order scan of
 * R_t = lam R_{t+1} + q_t do_t^T.
 *
 * Tensors.  Device pointers to contiguous row-major [B, H, T, d] (q, k, dq,
 * dk) and [B, H, T, d_v] (v, o, dout, dv) arrays of one element type `dtype`,
 * each 16-byte aligned.  Outputs have the input dtype; accumulation is fp32.
 * `decay` is a device pointer to H fp32 values in (0, 1], or NULL for lam = 1;
 * its values are read on the device and not validated (values outside (0, 1]
 * give unspecified results).
 *
 * Supported: d, d_v in {64, 128}; dtype LA2_BF16 or LA2_F32; block in
 * {16, 32, 64, 128, 256} for both.  `block` is the tile length asked for: the
 * split into intra- and inter-tile parts holds for every tile length (same
 * page, section 2), so the kernels run the nearest tile length they are built
 * for, with the state handed over between tiles, and the result is the same
 * up to rounding.  bf16 output scans run 64-position tiles for block 16, 32
 * and 64 and 128-position tiles for 128 and 256 (a 256 tile's Q, K and V
 * alone would fill the 160 KiB of LDS at d = 128); fp32 scans run 16, 32 or
 * 64 positions (64 for 128 and 256).  The bf16 backward with d = d_v computes
 * dK and dV in one fused reverse pass over 64-position tiles; without decay at
 * d = d_v = 128, la2_backward_saved computes dQ, dK and dV in one reverse pass.
 *
 * Ownership.  The caller allocates and frees every buffer, including the
 * workspace (la2_workspace_bytes tells its size; it may be 0, in which case
 * workspace may be NULL).  The library allocates nothing, never synchronizes,
 * keeps no state between calls and is safe to call from several threads.
 *
 * Execution.  Work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns at once.  Outputs and workspace are in use
 * until the stream reaches that point.
 *
 * Errors.  Every entry point returns LA2_OK (0) or a status below.  All
 * argument checks run before anything is enqueued, so a non-zero status other
 * than LA2_ERR_HIP means nothing was launched.  Nothing is printed and
 * nothing aborts.
 */
#ifndef LA2_H
#define LA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA2_ABI_VERSION 9

enum la2_dtype { LA2_F32 = 0, LA2_BF16 = 1 };

/* Feature maps of the normalized forward (la2_forward_normalized). */
enum la2_feature_map {
    LA2_PHI_IDENTITY = 0,   /* phi(x) = x */
    LA2_PHI_ELU1 = 1        /* phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise (strictly positive) */
};

enum la2_status {
    LA2_OK = 0,
    LA2_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    LA2_ERR_BAD_SHAPE = 2,           /* B, H, T, d or d_v <= 0, or sizes overflow */
    LA2_ERR_UNSUPPORTED = 3,         /* d / d_v / block / dtype outside the compiled set */
    LA2_ERR_MISALIGNED = 4,          /* a tensor pointer is not 16-byte aligned */
    LA2_ERR_ALIAS = 5,               /* an output overlaps an input, another output or the workspace */
    LA2_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes < la2_workspace_bytes(...) or NULL workspace */
    LA2_ERR_HIP = 7,                 /* a kernel launch failed (hipGetLastError) */
    LA2_ERR_SCRATCH_TOO_SMALL = 8    /* la2_forward_noalloc: the sizes need more than its static scratch */
};

/* Bytes of the static device scratch of la2_forward_noalloc (per GPU). */
#define LA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Forward: o = attention(q, k, v).
 *   q, k: [B, H, T, d]; v, o: [B, H, T, d_v]; decay: [H] fp32 or NULL.
 *   block: tile length T_B; dtype: enum la2_dtype.
 *   workspace: device scratch of at least la2_workspace_bytes(..., 0) bytes,
 *   used for the per-segment states when a chain is split across workgroups.
 *   On completion those bytes hold the state each segment starts from, which
 *   la2_backward_saved can reuse.  Without decay, with dtype LA2_BF16 and
 *   d = d_v = 128, a workspace of at least la2_workspace_bytes(..., 1) bytes
 *   also receives each chain's final state (fp32 [B, H, d, d_v], right after
 *   the segment states), from which la2_backward_saved walks the sequence
 *   backwards in one pass. */
int la2_forward(const void *q, const void *k, const void *v, const float *decay, void *o,
                int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/* la2_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same o as
 * la2_forward (the same kernels and plan), with no workspace argument: the
 * segment states of split chains live in a static device array of
 * LA2_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, which each
 * GPU holds from the first call on it until the process ends.  The call uses
 * the array of the current device (hipGetDevice); `stream` must belong to that
 * device.  It calls no hipMalloc or hipFree, and no allocating routine.
 *   The plan is la2_forward's, except that the state pass of split chains
 *   cuts a segment into no more pieces than the scratch holds states for (the
 *   result differs from la2_forward's only by rounding where that limit
 *   applies); the automatic plan then always fits, since one piece per segment
 *   needs at most 256 states of d x d_v <= 128 x 128 fp32 = 16 MiB.  Sizes
 *   whose plan would still need more (only forced plans of a test build) are
 *   rejected with LA2_ERR_SCRATCH_TOO_SMALL before anything is enqueued.
 *   All calls on one GPU share its array, and it keeps the last call's states:
 *   calls that overlap in time on one GPU (other streams, other threads, graph
 *   replays in flight together) race on it and give wrong results.  Calls
 *   ordered on one stream are safe.  Other arguments and errors as in
 *   la2_forward. */
int la2_forward_noalloc(const void *q, const void *k, const void *v, const float *decay, void *o,
                        int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype,
                        void *stream);

/* Forward carried in from and out to a state: the same o, for a sequence whose
 * prefix is summarized by state_in, and the state after its last position.
 * The state is the fixed-size summary of everything before a position (page
 * "Lightning Attention", section 2, "Memory footprint": the only persistent
 * state across tiles is the d x d_v matrix S), so splitting a sequence
 * anywhere and passing the state on gives the same outputs (chunked prefill,
 * exact resume):
 *     S_{-1} = state_in (0 when NULL),  S_t = lam S_{t-1} + k_t v_t^T,
 *     o_t = S_t^T q_t,  state_out = S_{T-1}.
 *   state_in, state_out: device fp32 [B, H, d, d_v], row-major (d rows), or
 *   NULL (start from zero / do not write the final state).  state_out may be
 *   the same pointer as state_in (updated in place) but may not otherwise
 *   overlap it, an input, o or the workspace.  Other arguments and the
 *   workspace as in la2_forward.  Its backward is la2_backward_state. */
int la2_forward_state(const void *q, const void *k, const void *v, const float *decay,
                      const float *state_in, void *o, float *state_out, int64_t B, int64_t H,
                      int64_t T, int64_t d, int64_t d_v, int block, int dtype, void *workspace,
                      size_t workspace_bytes, void *stream);

/* One generated token per chain (inference): state <- lam state + k v^T, then
 * o = state^T q, with the cost of one step whatever the length of the prefix
 * the state summarizes (Lightning Attention-2 abstract, arXiv 2401.04658:
 * constant speed at any length).
 *   q, k: [B, H, d]; v, o: [B, H, d_v] (one position, `dtype`); decay: [H] fp32
 *   or NULL; state: device fp32 [B, H, d, d_v], read and overwritten in place.
 *   o may not overlap an input or the state, nor the state an input.
 *   No workspace; supported d, d_v in {64, 128}. */
int la2_decode_step(const void *q, const void *k, const void *v, const float *decay, void *o,
                    float *state, int64_t B, int64_t H, int64_t d, int64_t d_v, int dtype,
                    void *stream);

/* Normalized forward: the whole output of page "Lightning Attention", section 1,
 * numerator over denominator, with a feature map applied to q and k and the
 * decay applied to both prefix sums:
 *     S_t = lam S_{t-1} + phi(k_t) v_t^T,   z_t = lam z_{t-1} + phi(k_t),
 *     o_t = S_t^T phi(q_t) / (z_t . phi(q_t)).
 *   feature_map: enum la2_feature_map.  With LA2_PHI_ELU1 every weight is
 *   positive, so o_t is a weighted average of v_0..v_t; with
 *   LA2_PHI_IDENTITY (the pages' default map) the denominator can vanish or
 *   change sign and is not guarded (a zero gives inf or NaN, as the formula
 *   does).  The denominator is accumulated first, in fp32 from phi in fp32;
 *   the numerator then runs through the same tiled scan as la2_forward (on
 *   phi(q), phi(k) rounded to `dtype`), each output row divided by its
 *   denominator in fp32 and rounded to `dtype` once when it is stored.
 *   Except in bf16 at d = d_v = 128 without decay, where the chains fill the
 *   GPU unsplit: there one launch reads q, k, v once and writes o, applying
 *   phi to the tiles in on-chip memory; numerator and denominator both come
 *   from phi(q), phi(k) rounded to bf16 (the denominator's sums in fp32), and
 *   with a workspace of la2_normalized_workspace_bytes(..., 1) bytes it also
 *   writes phi(q), phi(k) and the denominators there for
 *   la2_backward_normalized_saved.
 *   Other arguments as in la2_forward; workspace: at least
 *   la2_normalized_workspace_bytes(..., 0) bytes (phi(q) and phi(k) for
 *   LA2_PHI_ELU1, one fp32 denominator per position, per-segment sums and
 *   the numerator's own workspace; never 0).  Its backward is
 *   la2_backward_normalized. */
int la2_forward_normalized(const void *q, const void *k, const void *v, const float *decay, void *o,
                           int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int feature_map,
                           int block, int dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Backward of la2_forward_normalized: gradients of <o, dout> with respect to
 * q, k and v, by the chain rule through the ratio (pq = phi(q), pk = phi(k)):
 *     dn_t = do_t / den_t,   dden_t = -(do_t . o_t) / den_t,
 *     d pq_t = S_t dn_t + dden_t z_t,
 *     d pk_t = R_t v_t + sum_{s >= t} lam^(s-t) dden_s pq_s,   dv_t = R_t^T pk_t,
 *     dq = d pq (.) phi'(q),   dk = d pk (.) phi'(k),
 * R the reverse state of the numerator with output gradient dn.  The two
 * terms of d pq largely cancel, so with dtype LA2_BF16 dq is formed from
 * phi(k) = m + kap (m the chain's mean of phi(k)): the bf16 tile scan runs over
 * the small kap, and the parts that cancel (built from m, the prefix sums of v
 * and kap and the exact do_t . o_t) are combined in fp32; equal to the formula
 * above in exact arithmetic.
 *   o: the output la2_forward_normalized returned for these inputs (read).
 *   The denominator and phi(q), phi(k) are recomputed; the numerator's part
 *   runs through the same passes as la2_backward.  Other arguments as in
 *   la2_forward_normalized; workspace: at least
 *   la2_normalized_workspace_bytes(..., 1) bytes. */
int la2_backward_normalized(const void *q, const void *k, const void *v, const float *decay,
                            const void *o, const void *dout, void *dq, void *dk, void *dv,
                            int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v,
                            int feature_map, int block, int dtype, void *workspace,
                            size_t workspace_bytes, void *stream);

/* la2_backward_normalized for the training step: the workspace must be the one
 * that la2_forward_normalized was just given for the same q, k, v, decay,
 * feature map, block and dtype (at least la2_normalized_workspace_bytes(..., 1)
 * bytes, since the backward needs the larger size), unchanged since.  phi(q),
 * phi(k), the denominators, their segment sums and the numerator's segment
 * states are then read from it instead of recomputed; the result is the same
 * as la2_backward_normalized's.  With a workspace the forward did not fill,
 * the gradients are garbage (there is no way to detect it). */
int la2_backward_normalized_saved(const void *q, const void *k, const void *v, const float *decay,
                                  const void *o, const void *dout, void *dq, void *dk, void *dv,
                                  int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v,
                                  int feature_map, int block, int dtype, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Workspace bytes needed by la2_forward_normalized (backward = 0) or
 * la2_backward_normalized (backward = 1) for these arguments; (size_t)-1 for
 * arguments they would reject. */
size_t la2_normalized_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v,
                                      int feature_map, int block, int dtype, int backward);

/* The same o as la2_forward, computed the way the recurrence is written: one
 * position after another (page "Lightning Attention", section 1, where the
 * serial loop's rank-1 updates are what the tiling of section 2 removes).
 * Provided to compare the two on the same GPU, not for use on the hot path:
 * each position costs 2 d d_v vector FMAs and a chain is one workgroup per
 * 64 value columns, so the work runs in parallel only across chains.
 *   Arguments as in la2_forward, without block and workspace; fp32 state.
 *   Supported: d, d_v in {64, 128}, LA2_BF16 or LA2_F32. */
int la2_forward_serial(const void *q, const void *k, const void *v, const float *decay, void *o,
                       int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int dtype,
                       void *stream);

/* Backward: gradients of <o, dout> with respect to q, k and v.
 *   dout, dv: [B, H, T, d_v]; dq, dk: [B, H, T, d]; other arguments as in la2_forward.
 *   workspace: at least la2_workspace_bytes(..., 1) bytes. */
int la2_backward(const void *q, const void *k, const void *v, const float *decay, const void *dout,
                 void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t T, int64_t d,
                 int64_t d_v, int block, int dtype, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Backward that reuses the states of a preceding la2_forward (the usual training
 * step: forward, then backward on the same q, k, v), instead of recomputing them
 * from k and v.  Same arguments and results as la2_backward (up to rounding),
 * with one more precondition: `workspace` is the pointer that the la2_forward
 * call on the same q, k, v, decay, sizes, block and dtype received, with
 * workspace_bytes of at least la2_workspace_bytes(..., 1) in both calls, and
 * the states that forward left there are unchanged since (this call leaves
 * them unchanged too, so it may be repeated).  The library cannot check this;
 * with other contents the gradients are wrong.
 * Without decay, with dtype LA2_BF16 and d = d_v = 128 it starts from each
 * chain's final state and walks the sequence once in reverse: the state before
 * a tile is the state after it minus that tile's k^T v (exact arithmetic of the
 * undecayed recurrence), so dq, dk and dv come from one read of q, k, v and
 * dout.  Otherwise it runs la2_backward's passes, with the forward's segment
 * start states in place of their recomputation. */
int la2_backward_saved(const void *q, const void *k, const void *v, const float *decay,
                       const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H,
                       int64_t T, int64_t d, int64_t d_v, int block, int dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Backward of la2_forward_state: the gradients of <o, dout> + <state_out, dstate_out> with
 * respect to q, k, v and the carried-in state, so that a sequence trained in chunks, each chunk's
 * forward carried in from the state the previous one left and its d(state_in) passed back as the
 * previous chunk's dstate_out, gets the gradients of the whole sequence.  By the chain rule
 * through S_t = lam S_{t-1} + k_t v_t^T (S_{-1} = state_in):
 *     dq_t = S_t do_t;   R_{T-1} = q_{T-1} do_{T-1}^T + dstate_out,
 *     R_t = lam R_{t+1} + q_t do_t^T;   dk_t = R_t v_t;   dv_t = R_t^T k_t;
 *     dstate_in = lam R_0.
 *   state_in, dstate_out: device fp32 [B, H, d, d_v] or NULL (zero); dstate_in: device fp32
 *   [B, H, d, d_v] or NULL (not written).  dstate_in may not overlap anything else; the inputs may
 *   overlap each other.  Other arguments and the workspace (la2_workspace_bytes(..., 1)) as in
 *   la2_backward; with both states NULL it computes what la2_backward does. */
int la2_backward_state(const void *q, const void *k, const void *v, const float *decay,
                       const float *state_in, const void *dout, const float *dstate_out, void *dq,
                       void *dk, void *dv, float *dstate_in, int64_t B, int64_t H, int64_t T,
                       int64_t d, int64_t d_v, int block, int dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Workspace bytes needed by la2_forward / la2_forward_state (backward = 0) or la2_backward,
 * la2_backward_saved and la2_backward_state (backward = 1) for these sizes; the backward size is never
 * smaller, so one workspace of that size serves a forward + backward step.
 * (size_t)-1 for arguments that la2_forward/la2_backward would reject. */
size_t la2_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block,
                           int dtype, int backward);

/* Static, human-readable text for a status code. */
const char *la2_status_string(int status);

/* LA2_ABI_VERSION of the built library. */
int la2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA2_H */
