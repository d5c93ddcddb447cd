// la2_norm.hip -- the normalized output: feature map and denominator.
//
// Page "Lightning Attention" (lizeman.github.io llm-arch-kb), section 1: the full output divides
// the numerator phi(q_t)^T S_t by phi(q_t)^T z_t, where z_t is the prefix sum of phi(k_s); with a
// per-head decay z follows the same recurrence as S:
//   z_t = lam z_{t-1} + phi(k_t),    den_t = phi(q_t) . z_t,    o_t = (S_t^T phi(q_t)) / den_t.
// The numerator is the plain tile scan run on phi(q), phi(k).  The denominator is a d-vector scan:
// 2 d flops per position against 2 d elements read, so it is a pure HBM stream done on the vector
// ALUs.  It runs first, reading q and k once: it writes phi(q) and phi(k) for the numerator scan
// (elu + 1 only) and den_t in fp32; after the numerator scan one elementwise pass divides o.
//
// Denominator kernel layout: one workgroup of 256 threads per (chain, segment) walks the segment in
// chunks of 64 positions.  Thread (c8, g) owns 8 consecutive feature dims (c8 of D/8) and a run of
// 64 / G consecutive positions (group g of G = 256 / (D/8)); the D/8 threads of a group are
// consecutive lanes, so a row is one contiguous 2D- or 4D-byte read and a dot product over d is a
// butterfly across those lanes.  Per chunk: each group forms its run's decayed sum, the groups'
// sums are chained in LDS (Horner with lam^(run length)), then each group rewalks its run from
// its carried-in z and forms den_t.  Chains with few rows of work are cut into segments whose
// start vectors come from a separate pass over the earlier segments' sums.
#include "la2_internal.h"

namespace la2 {
namespace {

constexpr int kThreadsN = 256;
constexpr int kChunkN = 64;

template <int FMAP>
__device__ __forceinline__ float phi(float x) {
    if constexpr (FMAP == 1)
        return x > 0.0f ? x + 1.0f : expf(x);   // elu(x) + 1
    else
        return x;
}

__device__ __forceinline__ void load8(const __bf16 *p, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        x[2 * m] = __uint_as_float(w[m] << 16);
        x[2 * m + 1] = __uint_as_float(w[m] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
}

// round to nearest even (finite inputs)
__device__ __forceinline__ unsigned bf16_bits(float x) {
    const unsigned u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void store8(__bf16 *p, const float (&x)[8]) {
    uint4 u;
    u.x = bf16_bits(x[0]) | (bf16_bits(x[1]) << 16);
    u.y = bf16_bits(x[2]) | (bf16_bits(x[3]) << 16);
    u.z = bf16_bits(x[4]) | (bf16_bits(x[5]) << 16);
    u.w = bf16_bits(x[6]) | (bf16_bits(x[7]) << 16);
    *reinterpret_cast<uint4 *>(p) = u;
}

__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// NORM: write den_t of every position of segment `seg` (and phi(q), phi(k) where asked for).
// !NORM: write the segment's own decayed sum of phi(k) (z at its last position, starting from
// zero) to zseg.
template <typename E, int D, int FMAP, bool NORM>
__global__ __launch_bounds__(kThreadsN) void denom_kernel(DenArgs p) {
    constexpr int CPR = D / 8;                  // threads per row (8 dims each)
    constexpr int G = kThreadsN / CPR;          // position groups
    constexpr int PPG = kChunkN / G;            // positions per group per chunk
    static_assert(PPG >= 1 && kChunkN % G == 0, "layout");
    __shared__ float part[G][D];
    __shared__ float zc[2][D];

    const int tid = threadIdx.x, c8 = tid % CPR, g = tid / CPR;
    const int nseg_here = NORM ? p.nseg : p.nseg - 1;
    const int chain = blockIdx.x / nseg_here, seg = blockIdx.x % nseg_here;
    const float l2 = p.decay ? log2f(p.decay[chain % p.H]) : 0.0f;
    const float lam = exp2f(l2);
    const float lamG = exp2f((float)PPG * l2);
    const int64_t s0 = (int64_t)seg * p.seg_len;
    const int64_t s1 = min(p.T, s0 + p.seg_len);
    const E *kc = static_cast<const E *>(p.k) + (int64_t)chain * p.T * D + c8 * 8;
    const E *qc = static_cast<const E *>(p.q) + (int64_t)chain * p.T * D + c8 * 8;
    const bool keep_phi = FMAP != 0 && p.pq != nullptr;
    E *pqc = keep_phi ? static_cast<E *>(p.pq) + (int64_t)chain * p.T * D + c8 * 8 : nullptr;
    E *pkc = keep_phi ? static_cast<E *>(p.pk) + (int64_t)chain * p.T * D + c8 * 8 : nullptr;
    float *denc = p.den + (int64_t)chain * p.T;

    // z before the segment: Horner over the earlier segments' sums, z <- lam^seg_len z + dz_j
    if (tid < D) {
        float z = 0.0f;
        if (NORM && seg > 0) {
            const float lamS = exp2f((float)p.seg_len * l2);
            const float *zs = p.zseg + (int64_t)chain * (p.nseg - 1) * D + tid;
            for (int j = 0; j < seg; ++j) z = fmaf(z, lamS, zs[(int64_t)j * D]);
        }
        zc[0][tid] = z;
    }
    __syncthreads();

    int buf = 0;
    for (int64_t c0 = s0; c0 < s1; c0 += kChunkN) {
        float kk[PPG][8];
        float qq[NORM ? PPG : 1][8];
#pragma unroll
        for (int i = 0; i < PPG; ++i) {
            const int64_t s = c0 + g * PPG + i;
            if (s < s1) {
                load8(kc + s * D, kk[i]);
                if constexpr (NORM) load8(qc + s * D, qq[i]);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    kk[i][m] = phi<FMAP>(kk[i][m]);
                    if constexpr (NORM) qq[i][m] = phi<FMAP>(qq[i][m]);
                }
                if constexpr (NORM && FMAP != 0) {
                    if (keep_phi) {
                        store8(pqc + s * D, qq[i]);
                        store8(pkc + s * D, kk[i]);
                    }
                }
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    kk[i][m] = 0.0f;
                    if constexpr (NORM) qq[i][m] = 0.0f;
                }
            }
        }
        // this run's decayed sum, z at its last position when starting from zero
        float loc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) loc[m] = kk[0][m];
#pragma unroll
        for (int i = 1; i < PPG; ++i)
#pragma unroll
            for (int m = 0; m < 8; ++m) loc[m] = fmaf(loc[m], lam, kk[i][m]);
#pragma unroll
        for (int m = 0; m < 8; ++m) part[g][c8 * 8 + m] = loc[m];
        __syncthreads();
        // z entering this run: the chunk's carry, then the earlier runs of the chunk
        float z[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) z[m] = zc[buf][c8 * 8 + m];
        for (int j = 0; j < g; ++j)
#pragma unroll
            for (int m = 0; m < 8; ++m) z[m] = fmaf(z[m], lamG, part[j][c8 * 8 + m]);
        if constexpr (NORM) {
#pragma unroll
            for (int i = 0; i < PPG; ++i) {
                float pd = 0.0f;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    z[m] = fmaf(z[m], lam, kk[i][m]);
                    pd = fmaf(z[m], qq[i][m], pd);
                }
#pragma unroll
                for (int w = 1; w < CPR; w <<= 1) pd += __shfl_xor(pd, w, CPR);
                const int64_t s = c0 + g * PPG + i;
                if (s < s1 && c8 == 0) denc[s] = pd;
            }
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) z[m] = fmaf(z[m], lamG, loc[m]);
        }
        // the last run's z is the next chunk's carry (only read when this chunk was full)
        if (g == G - 1)
#pragma unroll
            for (int m = 0; m < 8; ++m) zc[buf ^ 1][c8 * 8 + m] = z[m];
        __syncthreads();
        buf ^= 1;
    }
    if constexpr (!NORM) {
        if (tid < D) p.zseg[((int64_t)chain * (p.nseg - 1) + seg) * D + tid] = zc[buf][tid];
    }
}

// o[r, :] /= den[r] over `rows` rows of DV elements.  Each thread takes 4 groups of 8 elements per
// step, 256 threads apart, and issues all their loads before the first division.
constexpr int kDivUnroll = 4;

template <typename E, int DV>
__global__ __launch_bounds__(kThreadsN) void divide_kernel(E *o, const float *den, int64_t rows) {
    constexpr int G8 = DV / 8;
    const int64_t n = rows * G8, stride = (int64_t)gridDim.x * kThreadsN * kDivUnroll;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreadsN * kDivUnroll + threadIdx.x; i0 < n; i0 += stride) {
        float x[kDivUnroll][8], d[kDivUnroll];
#pragma unroll
        for (int u = 0; u < kDivUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * kThreadsN;
            if (i < n) {
                load8(o + i * 8, x[u]);
                d[u] = den[i / G8];
            }
        }
#pragma unroll
        for (int u = 0; u < kDivUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * kThreadsN;
            if (i < n) {
#pragma unroll
                for (int m = 0; m < 8; ++m) x[u][m] = x[u][m] / d[u];
                store8(o + i * 8, x[u]);
            }
        }
    }
}

template <typename E, int D, int FMAP>
hipError_t launch_den(const DenArgs &a, bool norm, hipStream_t s) {
    const unsigned grid = (unsigned)a.chains * (unsigned)(norm ? a.nseg : a.nseg - 1);
    if (norm)
        hipLaunchKernelGGL((denom_kernel<E, D, FMAP, true>), dim3(grid), dim3(kThreadsN), 0, s, a);
    else
        hipLaunchKernelGGL((denom_kernel<E, D, FMAP, false>), dim3(grid), dim3(kThreadsN), 0, s, a);
    return hipGetLastError();
}

template <typename E, int FMAP>
hipError_t launch_den_e(const DenArgs &a, int D, bool norm, hipStream_t s) {
    return D == 64 ? launch_den<E, 64, FMAP>(a, norm, s) : launch_den<E, 128, FMAP>(a, norm, s);
}

template <typename E>
hipError_t launch_div_e(void *o, const float *den, int64_t rows, int DV, hipStream_t s) {
    const int64_t want = (rows * (DV / 8) + kThreadsN * kDivUnroll - 1) / (kThreadsN * kDivUnroll);
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    if (DV == 64)
        hipLaunchKernelGGL((divide_kernel<E, 64>), dim3(grid), dim3(kThreadsN), 0, s, static_cast<E *>(o), den, rows);
    else
        hipLaunchKernelGGL((divide_kernel<E, 128>), dim3(grid), dim3(kThreadsN), 0, s, static_cast<E *>(o), den, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_denominator(const DenArgs &a, int D, int dtype, int fmap, bool norm, hipStream_t s) {
    if (!(D == 64 || D == 128) || a.chains <= 0 || a.nseg < (norm ? 1 : 2) || a.seg_len % kChunkN != 0 ||
        (fmap != 0 && fmap != 1))
        return hipErrorInvalidValue;
    if (dtype == 1)
        return fmap ? launch_den_e<__bf16, 1>(a, D, norm, s) : launch_den_e<__bf16, 0>(a, D, norm, s);
    return fmap ? launch_den_e<float, 1>(a, D, norm, s) : launch_den_e<float, 0>(a, D, norm, s);
}

hipError_t launch_divide(void *o, const float *den, int64_t rows, int DV, int dtype, hipStream_t s) {
    if (!(DV == 64 || DV == 128) || rows <= 0) return hipErrorInvalidValue;
    return dtype == 1 ? launch_div_e<__bf16>(o, den, rows, DV, s) : launch_div_e<float>(o, den, rows, DV, s);
}

}  // namespace la2
