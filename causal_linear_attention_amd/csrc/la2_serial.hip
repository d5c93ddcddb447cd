// la2_serial.hip -- the token-serial recurrence, for comparison with the tiled scan.
//
// Page "Lightning Attention" (lizeman.github.io llm-arch-kb), section 1: run as written, the
// recurrence S_t = lam S_{t-1} + k_t v_t^T, o_t = S_t^T q_t is serial in t and every step is a
// rank-1 update, so it cannot use matrix cores and its parallelism is only chains x d x d_v.  This
// kernel is that loop done as well as the vector ALUs allow: one workgroup of 4 waves per (chain,
// 64-wide value slice) keeps the fp32 state in registers (lane = value column, wave = a quarter of
// the d rows), stages q, k, v through LDS in chunks of 16 positions (coalesced reads, one barrier
// per chunk), and reduces the 4 waves' partial outputs per chunk.  Each position costs 2 d d_v
// FMAs on the vector ALUs; the tiled scan does the same work as dense MFMA products.
#include "la2_internal.h"

namespace la2 {
namespace {

constexpr int kThreadsS = 256;
constexpr int kChunkS = 16;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

template <typename E, int D>
__global__ __launch_bounds__(kThreadsS) void serial_kernel(const E *q, const E *k, const E *v, const float *decay,
                                                           E *o, int64_t T, int H, int DVT) {
    constexpr int R = D / 4;   // state rows per thread
    __shared__ __attribute__((aligned(16))) float sq[kChunkS][D];
    __shared__ __attribute__((aligned(16))) float sk[kChunkS][D];
    __shared__ float sv[kChunkS][64];
    __shared__ float po[kChunkS][4][64];

    const int nslice = DVT / 64;
    const int chain = blockIdx.x / nslice, dv0 = (blockIdx.x % nslice) * 64;
    const int tid = threadIdx.x, c = tid & 63, w = tid >> 6;
    const float lam = decay ? decay[chain % H] : 1.0f;
    const E *qc = q + (int64_t)chain * T * D, *kc = k + (int64_t)chain * T * D;
    const E *vc = v + (int64_t)chain * T * DVT + dv0;
    E *oc = o + (int64_t)chain * T * DVT + dv0;

    float S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) S[r] = 0.0f;

    for (int64_t c0 = 0; c0 < T; c0 += kChunkS) {
        const int n = (int)min((int64_t)kChunkS, T - c0);
        for (int e = tid; e < kChunkS * D; e += kThreadsS) {
            const int t = e / D, i = e % D;
            sq[t][i] = t < n ? to_f(qc[(c0 + t) * D + i]) : 0.0f;
            sk[t][i] = t < n ? to_f(kc[(c0 + t) * D + i]) : 0.0f;
        }
        for (int e = tid; e < kChunkS * 64; e += kThreadsS) {
            const int t = e / 64, j = e % 64;
            sv[t][j] = t < n ? to_f(vc[(c0 + t) * DVT + j]) : 0.0f;
        }
        __syncthreads();
        for (int t = 0; t < n; ++t) {
            const float vt = sv[t][c];
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                S[r] = fmaf(lam, S[r], sk[t][w * R + r] * vt);
                acc = fmaf(S[r], sq[t][w * R + r], acc);
            }
            po[t][w][c] = acc;
        }
        __syncthreads();
        for (int e = tid; e < n * 64; e += kThreadsS) {
            const int t = e / 64, j = e % 64;
            oc[(c0 + t) * DVT + j] = from_f<E>((po[t][0][j] + po[t][1][j]) + (po[t][2][j] + po[t][3][j]));
        }
        // the next chunk's staging rewrites sq, sk, sv only after this barrier; po is rewritten
        // only after the next one
        __syncthreads();
    }
}

template <typename E>
hipError_t launch_serial_e(const void *q, const void *k, const void *v, const float *decay, void *o, int chains,
                           int H, int64_t T, int D, int DV, hipStream_t s) {
    const unsigned grid = (unsigned)chains * (unsigned)(DV / 64);
    if (D == 64)
        hipLaunchKernelGGL((serial_kernel<E, 64>), dim3(grid), dim3(kThreadsS), 0, s, static_cast<const E *>(q),
                           static_cast<const E *>(k), static_cast<const E *>(v), decay, static_cast<E *>(o), T, H, DV);
    else
        hipLaunchKernelGGL((serial_kernel<E, 128>), dim3(grid), dim3(kThreadsS), 0, s, static_cast<const E *>(q),
                           static_cast<const E *>(k), static_cast<const E *>(v), decay, static_cast<E *>(o), T, H, DV);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_serial(const void *q, const void *k, const void *v, const float *decay, void *o, int chains, int H,
                         int64_t T, int D, int DV, int dtype, hipStream_t s) {
    if (!((D == 64 || D == 128) && (DV == 64 || DV == 128)) || chains <= 0 || T <= 0) return hipErrorInvalidValue;
    return dtype == 1 ? launch_serial_e<__bf16>(q, k, v, decay, o, chains, H, T, D, DV, s)
                      : launch_serial_e<float>(q, k, v, decay, o, chains, H, T, D, DV, s);
}

}  // namespace la2
