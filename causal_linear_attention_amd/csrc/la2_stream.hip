// la2_stream.hip -- a plain HBM stream for measurement (test build only): the ceiling the tile kernels'
// read:write mixes can reach on this GPU with 16-byte lane accesses.
//
// dst_j[i] = src_0[i] + ... + src_{n-1}[i] (u32 lanes, wrapping) for every 16-byte chunk i of `bytes`,
// so every source byte is read once and every destination byte written once per launch; a grid-stride
// loop over the chunks with `blocks` workgroups of `threads` threads, with or without the nontemporal
// cache hint (the policy of the bf16 kernels' tile loads and stores).
//
// la2_test_reread: whether a second read of the same bytes, shortly after the first, is served by the
// memory-side cache.  Four same-sized buffers q, k, v, o are cut into items of item_bytes; one
// workgroup of 512 threads per item (with 144 KiB of LDS, so one per CU, as the tile kernels run):
//   phase A  reads the item's k and v (the state-only pass of a split chain),
//   phase B  reads its q, k, v and writes o = q ^ k ^ v (^ A's result: the output pass).
// Mode 0 runs B alone, mode 1 A then B in one workgroup (A's loads with the default cache policy so
// that B can hit), mode 2 A alone.
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

constexpr int kRereadThreads = 512;
constexpr size_t kRereadLds = 144 * 1024;

template <int MODE>
__global__ __launch_bounds__(kRereadThreads) void reread_kernel(const u32x4 *q, const u32x4 *k, const u32x4 *v,
                                                                u32x4 *o, u32x4 *sink, int64_t item_chunks,
                                                                bool nt) {
    extern __shared__ u32x4 lds_pad[];
    const int64_t base = (int64_t)blockIdx.x * item_chunks;
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (MODE >= 1) {
        for (int64_t j = threadIdx.x; j < item_chunks; j += kRereadThreads) {
            const u32x4 a = MODE == 1 || !nt ? k[base + j] : __builtin_nontemporal_load(k + base + j);
            const u32x4 b = MODE == 1 || !nt ? v[base + j] : __builtin_nontemporal_load(v + base + j);
            acc ^= a ^ b;
        }
    }
    if (MODE <= 1) {
        for (int64_t j = threadIdx.x; j < item_chunks; j += kRereadThreads) {
            u32x4 x = nt ? __builtin_nontemporal_load(q + base + j) : q[base + j];
            x ^= nt ? __builtin_nontemporal_load(k + base + j) : k[base + j];
            x ^= nt ? __builtin_nontemporal_load(v + base + j) : v[base + j];
            if (nt)
                __builtin_nontemporal_store(x ^ acc, o + base + j);
            else
                o[base + j] = x ^ acc;
        }
    } else {
        // A alone: one 16-byte result per workgroup keeps its loads live
        if (threadIdx.x == 0) sink[blockIdx.x] = acc;
    }
    if (threadIdx.x == 0) lds_pad[0] = acc;
}

template <int MODE>
hipError_t launch_reread(const u32x4 *q, const u32x4 *k, const u32x4 *v, u32x4 *o, int64_t items,
                         int64_t item_chunks, bool nt, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(reread_kernel<MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRereadLds);
    if (e != hipSuccess) return e;
    // mode 2 writes one chunk per item: into o, which it does not otherwise touch
    hipLaunchKernelGGL(reread_kernel<MODE>, dim3((unsigned)items), dim3(kRereadThreads), kRereadLds, s, q, k, v, o,
                       o, item_chunks, nt);
    return hipGetLastError();
}

}  // namespace

extern "C" int la2_test_reread(const void *q, const void *k, const void *v, void *o, size_t bytes, size_t item_bytes,
                               int mode, int nontemporal, void *stream) {
    if (bytes == 0 || item_bytes == 0 || item_bytes % 16 || bytes % item_bytes || bytes / item_bytes > 0x7fffffff ||
        mode < 0 || mode > 2)
        return 2;   // LA2_ERR_BAD_SHAPE
    for (const void *p : {q, k, v, static_cast<const void *>(o)})
        if (!p || (reinterpret_cast<uintptr_t>(p) & 15u)) return 1;
    const auto *q4 = static_cast<const u32x4 *>(q), *k4 = static_cast<const u32x4 *>(k);
    const auto *v4 = static_cast<const u32x4 *>(v);
    auto *o4 = static_cast<u32x4 *>(o);
    const int64_t items = (int64_t)(bytes / item_bytes), item_chunks = (int64_t)(item_bytes / 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool nt = nontemporal != 0;
    hipError_t e = mode == 0   ? launch_reread<0>(q4, k4, v4, o4, items, item_chunks, nt, s)
                   : mode == 1 ? launch_reread<1>(q4, k4, v4, o4, items, item_chunks, nt, s)
                               : launch_reread<2>(q4, k4, v4, o4, items, item_chunks, nt, s);
    return e == hipSuccess ? 0 : 7;   // LA2_ERR_HIP
}

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
