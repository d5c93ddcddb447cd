// la2_stream.hip -- a plain HBM stream for measurement (test build only): the ceiling the tile kernels'
// read:write mixes can reach on this GPU with 16-byte lane accesses.
//
// dst_j[i] = src_0[i] + ... + src_{n-1}[i] (u32 lanes, wrapping) for every 16-byte chunk i of `bytes`,
// so every source byte is read once and every destination byte written once per launch; a grid-stride
// loop over the chunks with `blocks` workgroups of `threads` threads, with or without the nontemporal
// cache hint (the policy of the bf16 kernels' tile loads and stores).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "la2_test_hooks.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxSrc = 4, kMaxDst = 3;

struct StreamArgs {
    const u32x4 *src[kMaxSrc];
    u32x4 *dst[kMaxDst];
    int64_t chunks;
};

template <int NS, int ND, bool NT>
__global__ void stream_kernel(StreamArgs a) {
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.chunks; i += step) {
        u32x4 acc = NT ? __builtin_nontemporal_load(a.src[0] + i) : a.src[0][i];
#pragma unroll
        for (int s = 1; s < NS; ++s) acc += NT ? __builtin_nontemporal_load(a.src[s] + i) : a.src[s][i];
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            if (NT)
                __builtin_nontemporal_store(acc, a.dst[d] + i);
            else
                a.dst[d][i] = acc;
        }
    }
}

template <int NS, int ND>
hipError_t launch_nd(const StreamArgs &a, int blocks, int threads, bool nt, hipStream_t s) {
    if (nt)
        hipLaunchKernelGGL((stream_kernel<NS, ND, true>), dim3(blocks), dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL((stream_kernel<NS, ND, false>), dim3(blocks), dim3(threads), 0, s, a);
    return hipGetLastError();
}

template <int NS>
hipError_t launch_ns(const StreamArgs &a, int ndst, int blocks, int threads, bool nt, hipStream_t s) {
    switch (ndst) {
        case 1: return launch_nd<NS, 1>(a, blocks, threads, nt, s);
        case 2: return launch_nd<NS, 2>(a, blocks, threads, nt, s);
        default: return launch_nd<NS, 3>(a, blocks, threads, nt, s);
    }
}

}  // namespace

extern "C" int la2_test_stream(const void *const *src, int nsrc, void *const *dst, int ndst, size_t bytes, int blocks,
                               int threads, int nontemporal, void *stream) {
    if (!src || !dst || nsrc < 1 || nsrc > kMaxSrc || ndst < 1 || ndst > kMaxDst || bytes == 0 || bytes % 16 ||
        blocks < 1 || threads < 64 || threads > 1024 || threads % 64)
        return 2;   // LA2_ERR_BAD_SHAPE
    StreamArgs a{};
    for (int i = 0; i < nsrc; ++i) {
        if (!src[i] || (reinterpret_cast<uintptr_t>(src[i]) & 15u)) return 1;
        a.src[i] = static_cast<const u32x4 *>(src[i]);
    }
    for (int i = 0; i < ndst; ++i) {
        if (!dst[i] || (reinterpret_cast<uintptr_t>(dst[i]) & 15u)) return 1;
        a.dst[i] = static_cast<u32x4 *>(dst[i]);
    }
    a.chunks = (int64_t)(bytes / 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (nsrc) {
        case 1: e = launch_ns<1>(a, ndst, blocks, threads, nontemporal != 0, s); break;
        case 2: e = launch_ns<2>(a, ndst, blocks, threads, nontemporal != 0, s); break;
        case 3: e = launch_ns<3>(a, ndst, blocks, threads, nontemporal != 0, s); break;
        default: e = launch_ns<4>(a, ndst, blocks, threads, nontemporal != 0, s); break;
    }
    return e == hipSuccess ? 0 : 7;   // LA2_ERR_HIP
}
