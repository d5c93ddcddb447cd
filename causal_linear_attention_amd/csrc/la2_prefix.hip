// la2_prefix.hip -- chain the per-segment states of a split sequence.
//
// When a chain is cut into segments that run on different workgroups, each segment
// first produces its own state delta (the state it would reach from zero), and this
// kernel turns the deltas into the state each segment starts from.  The state is the
// fixed-size summary of everything before the segment (page "Lightning Attention",
// lizeman.github.io llm-arch-kb, section 2, "Memory footprint": the only persistent
// state across tiles is the d x d_v matrix S), so the hand-over is one affine step
// per segment:
//   forward: S_in[0] = init (0 if none),  S_in[p+1] = lam^L S_in[p] + dS[p]
//   reverse: R_in[last] = init (0 if none),  R_in[p-1] = lam^L R_in[p] + dR[p]
// L is the segment length in positions (every segment except the last is full).  A reverse
// init is the gradient of a carried-out forward state, attached at the chain's last position
// rather than one past the last segment's end, so the first reverse step multiplies it by
// lam^init_len instead (init_len = the last segment's length - 1).
#include "la2_internal.h"

namespace la2 {
namespace {

constexpr int kBatch = 8;

__global__ __launch_bounds__(256) void segment_prefix_kernel(float *states, const float *decay, int H, int nseg,
                                                             int64_t seg_len, int64_t elems, int reverse,
                                                             const float *init, int64_t init_len) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int chain = blockIdx.y;
    if (e >= elems) return;
    const float l2 = decay ? log2f(decay[chain % H]) : 0.0f;
    const float f = decay ? exp2f((float)seg_len * l2) : 1.0f;
    float *base = states + (int64_t)chain * nseg * elems + e;
    float run = init ? init[(int64_t)chain * elems + e] : 0.0f;
    // The deltas are read kBatch at a time before any of them is overwritten, so their loads are in
    // flight together rather than one segment's latency after another.
    if (!reverse) {
        for (int p0 = 0; p0 < nseg; p0 += kBatch) {
            float d[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) d[i] = p0 + i < nseg - 1 ? base[(int64_t)(p0 + i) * elems] : 0.0f;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (p0 + i < nseg) {
                    base[(int64_t)(p0 + i) * elems] = run;
                    run = fmaf(f, run, d[i]);
                }
            }
        }
    } else {
        const float f0 = init && decay ? exp2f((float)init_len * l2) : f;
        for (int p0 = nseg - 1; p0 >= 0; p0 -= kBatch) {
            float d[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) d[i] = p0 - i > 0 ? base[(int64_t)(p0 - i) * elems] : 0.0f;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int p = p0 - i;
                if (p >= 0) {
                    base[(int64_t)p * elems] = run;
                    run = fmaf(p == nseg - 1 ? f0 : f, run, d[i]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_segment_prefix(float *states, const float *decay, int chains, int H, int nseg, int64_t seg_len,
                                 int64_t elems, Dir dir, hipStream_t s, const float *init, int64_t init_len) {
    dim3 grid((unsigned)((elems + 255) / 256), (unsigned)chains);
    hipLaunchKernelGGL(segment_prefix_kernel, grid, dim3(256), 0, s, states, decay, H, nseg, seg_len, elems,
                       dir == Dir::Reverse ? 1 : 0, init, init_len);
    return hipGetLastError();
}

}  // namespace la2
