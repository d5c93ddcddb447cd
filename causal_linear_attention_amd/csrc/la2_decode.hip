// la2_decode.hip -- one generated token of causal linear attention per chain (inference).
//
// With the state carried as the summary of the whole prefix (page "Lightning Attention",
// lizeman.github.io llm-arch-kb, section 2, "Memory footprint": the only persistent state is the
// d x d_v matrix S; Lightning Attention-2 abstract, arXiv 2401.04658: constant speed whatever the
// length), a new token costs one step of the recurrence, independent of how long the prefix was:
//   S <- lam S + k v^T,   o = S^T q.
// The step is a pure stream over S (read and written once, fp32) with two dot-product-sized
// operands, so it is HBM-bound and uses plain FMAs, not MFMA.  One workgroup of 4 waves owns a
// 64-column slice of one chain's S: lane l holds column l of the slice, wave w rows
// [w D/4, (w+1) D/4); each row access is 64 consecutive floats (256 B).  The four partial dot
// products meet in LDS.  When the states together exceed the 256 MiB memory-side cache they are
// streamed with the nontemporal hint (nothing of them survives to the next step anyway); smaller
// sets keep the default policy, which leaves them cache-resident from one step to the next.
#include "la2_internal.h"

namespace la2 {
namespace {

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename E, int D, int DV, bool STREAM>
__global__ __launch_bounds__(256) void decode_kernel(const E *q, const E *k, const E *v, const float *decay, E *o,
                                                     float *state, int H) {
    constexpr int NSL = DV / 64, R = D / 4;
    const int chain = blockIdx.x / NSL, n = (blockIdx.x % NSL) * 64 + (threadIdx.x & 63);
    const int wave = threadIdx.x >> 6;
    const float lam = decay ? decay[chain % H] : 1.0f;
    const E *qc = q + (int64_t)chain * D, *kc = k + (int64_t)chain * D;
    const float vn = to_f32(v[(int64_t)chain * DV + n]);
    float *Sc = state + (int64_t)chain * D * DV + n;
    float acc = 0.0f;
#pragma unroll 8
    for (int r = 0; r < R; ++r) {
        const int i = wave * R + r;
        float *const p = Sc + (int64_t)i * DV;
        const float s = fmaf(lam, STREAM ? __builtin_nontemporal_load(p) : *p, to_f32(kc[i]) * vn);
        if constexpr (STREAM)
            __builtin_nontemporal_store(s, p);
        else
            *p = s;
        acc = fmaf(s, to_f32(qc[i]), acc);
    }
    __shared__ float red[4][64];
    red[wave][threadIdx.x & 63] = acc;
    __syncthreads();
    if (wave == 0) {
        const int l = threadIdx.x;
        o[(int64_t)chain * DV + n] = from_f32<E>((red[0][l] + red[1][l]) + (red[2][l] + red[3][l]));
    }
}

template <typename E, int D, int DV>
void launch_policy(const void *q, const void *k, const void *v, const float *decay, void *o, float *state,
                   int chains, int H, hipStream_t s) {
    constexpr int64_t kCacheBytes = (int64_t)256 << 20;
    const unsigned grid = (unsigned)chains * (unsigned)(DV / 64);
    const bool stream = (int64_t)chains * D * DV * (int64_t)sizeof(float) > kCacheBytes;
    if (stream)
        hipLaunchKernelGGL((decode_kernel<E, D, DV, true>), dim3(grid), dim3(256), 0, s, static_cast<const E *>(q),
                           static_cast<const E *>(k), static_cast<const E *>(v), decay, static_cast<E *>(o), state, H);
    else
        hipLaunchKernelGGL((decode_kernel<E, D, DV, false>), dim3(grid), dim3(256), 0, s, static_cast<const E *>(q),
                           static_cast<const E *>(k), static_cast<const E *>(v), decay, static_cast<E *>(o), state, H);
}

template <typename E, int D>
hipError_t launch_dv(const void *q, const void *k, const void *v, const float *decay, void *o, float *state,
                     int chains, int H, int DV, hipStream_t s) {
    if (DV == 64)
        launch_policy<E, D, 64>(q, k, v, decay, o, state, chains, H, s);
    else
        launch_policy<E, D, 128>(q, k, v, decay, o, state, chains, H, s);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const void *q, const void *k, const void *v, const float *decay, void *o, float *state,
                    int chains, int H, int D, int DV, hipStream_t s) {
    return D == 64 ? launch_dv<E, 64>(q, k, v, decay, o, state, chains, H, DV, s)
                   : launch_dv<E, 128>(q, k, v, decay, o, state, chains, H, DV, s);
}

}  // namespace

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *decay, void *o, float *state,
                         int chains, int H, int D, int DV, int dtype, hipStream_t s) {
    if (!((D == 64 || D == 128) && (DV == 64 || DV == 128)) || chains <= 0) return hipErrorInvalidValue;
    return dtype == 1 ? launch_e<__bf16>(q, k, v, decay, o, state, chains, H, D, DV, s)
                      : launch_e<float>(q, k, v, decay, o, state, chains, H, D, DV, s);
}

}  // namespace la2
