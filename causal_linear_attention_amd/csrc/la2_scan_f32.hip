// la2_scan_f32.hip -- fp32 tile-scan kernel (true fp32 arithmetic, no reduced-precision modes).
//
// Same decomposition as the bf16 MFMA kernel (page "Lightning Attention",
// lizeman.github.io llm-arch-kb, section 2, Steps 1-4), done with plain fp32 FMAs
// out of LDS.  One workgroup owns one (chain, segment, 64-wide value slice); per tile:
//   P   = (Q_b K_b^T) (.) mask      (Step 2 scores with the causal decay mask)
//   O_b = diag(w_inter) Q_b S + P V_b
//   S   = lam^TB S + (diag(w_upd) K_b)^T V_b
// with the forward / reverse weights documented in la2_scan_bf16.hip.
#include "la2_internal.h"

namespace la2 {
namespace {

constexpr int kThreads = 256;

template <int D, int DV, int TB, Dir DIR, Mode MODE>
__global__ __launch_bounds__(kThreads) void scan_f32_kernel(ScanArgs p) {
    constexpr bool kOut = MODE == Mode::Output;
    __shared__ float sQ[kOut ? TB * D : 1];
    __shared__ float sK[TB * D];
    __shared__ float sV[TB * DV];
    __shared__ float sP[kOut ? TB * TB : 1];
    __shared__ float sS[D * DV];
    static_assert(((kOut ? 2 * TB * D + TB * TB : TB * D) + TB * DV + D * DV) * 4 <= 160 * 1024, "LDS");

    const int tid = threadIdx.x;
    int item = blockIdx.x;
    const int slice = item % p.nslice;
    item /= p.nslice;
    const int seg = p.seg_first + item % p.seg_count;
    const int chain = item / p.seg_count;
    const int dv0 = slice * DV;
    const int64_t T = p.T;
    const int64_t NT = (T + TB - 1) / TB;
    const int64_t tile_lo = (int64_t)seg * p.seg_tiles;
    const int64_t tile_hi = min(tile_lo + p.seg_tiles, NT);
    if (tile_lo >= tile_hi) return;
    const int ntiles = (int)(tile_hi - tile_lo);

    const float *ga = static_cast<const float *>(p.a) + (int64_t)chain * T * D;
    const float *gb = static_cast<const float *>(p.b) + (int64_t)chain * T * D;
    const float *gc = static_cast<const float *>(p.c) + (int64_t)chain * T * p.DVT + dv0;
    float *gy = kOut ? static_cast<float *>(p.y) + (int64_t)chain * T * p.DVT + dv0 : nullptr;
    const int sidx = state_index(seg, p.sub, p.nsub, DIR == Dir::Reverse);
    float *gs = p.states ? p.states + ((int64_t)chain * p.nsub + sidx) * D * p.DVT + (p.states_t ? (int64_t)dv0 * D : dv0)
                         : nullptr;

    const bool has_decay = p.decay != nullptr;
    const float l2 = has_decay ? log2f(p.decay[chain % p.H]) : 0.0f;
    auto pw = [&](int n) -> float { return has_decay ? exp2f((float)n * l2) : 1.0f; };

    const bool init_state = kOut && gs != nullptr &&
                            (DIR == Dir::Forward ? (seg > 0 || p.has_init) : (seg < p.nseg - 1 || p.has_init));
    // reverse with a carried-in state: attached at the chain's last position (weights lam^(leff-1-i)
    // and carry lam^(leff-1) on the chain's last tile, the first this workgroup processes)
    const bool end_init = DIR == Dir::Reverse && kOut && p.has_init && seg == p.nseg - 1;
    const int leff_end = (int)min((int64_t)TB, T - (NT - 1) * TB);
    for (int e = tid; e < D * DV; e += kThreads)
        sS[e] = init_state ? gs[p.states_t ? (int64_t)(e % DV) * D + e / DV : (int64_t)(e / DV) * p.DVT + e % DV] : 0.0f;

    for (int it = 0; it < ntiles; ++it) {
        const int64_t t0 = (DIR == Dir::Forward ? tile_lo + it : tile_hi - 1 - it) * TB;
        const bool update = (MODE == Mode::StateOnly) || (it + 1 < ntiles);
        __syncthreads();   // previous tile fully consumed
        for (int e = tid; e < TB * D; e += kThreads) {
            const int64_t t = t0 + e / D;
            const float kv = t < T ? gb[t * D + e % D] : 0.0f;
            sK[e] = kv;
            if constexpr (kOut) sQ[e] = t < T ? ga[t * D + e % D] : 0.0f;
        }
        for (int e = tid; e < TB * DV; e += kThreads) {
            const int64_t t = t0 + e / DV;
            sV[e] = t < T ? gc[t * p.DVT + e % DV] : 0.0f;
        }
        __syncthreads();

        if constexpr (kOut) {
            // Step 2 scores with the causal decay mask
            for (int e = tid; e < TB * TB; e += kThreads) {
                const int i = e / TB, j = e % TB;
                const int diff = DIR == Dir::Forward ? i - j : j - i;
                float acc = 0.0f;
                if (diff >= 0) {
                    for (int c = 0; c < D; ++c) acc = fmaf(sQ[i * D + c], sK[j * D + c], acc);
                    acc *= pw(diff);
                }
                sP[e] = acc;
            }
            __syncthreads();
            // Step 3 + Step 2 output
            for (int e = tid; e < TB * DV; e += kThreads) {
                const int i = e / DV, n = e % DV;
                float inter = 0.0f;
                for (int c = 0; c < D; ++c) inter = fmaf(sQ[i * D + c], sS[c * DV + n], inter);
                int ew = DIR == Dir::Forward ? i + 1 : TB - i;
                if (end_init && it == 0) ew = leff_end - 1 - i;
                float acc = ew >= 0 ? inter * pw(ew) : 0.0f;
                for (int j = 0; j < TB; ++j) acc = fmaf(sP[i * TB + j], sV[j * DV + n], acc);
                const int64_t t = t0 + i;
                if (t < T) gy[t * p.DVT + n] = p.den ? acc / p.den[(int64_t)chain * T + t] : acc;
            }
            __syncthreads();   // sS reads done before the update
        }
        // Step 4 state update
        if (update) {
            const float f = (end_init && it == 0) ? pw(leff_end - 1) : pw(TB);
            for (int e = tid; e < D * DV; e += kThreads) {
                const int c = e / DV, n = e % DV;
                float acc = sS[e] * f;
                for (int j = 0; j < TB; ++j)
                    acc = fmaf(sK[j * D + c] * pw(DIR == Dir::Forward ? TB - 1 - j : j), sV[j * DV + n], acc);
                sS[e] = acc;
            }
        }
    }
    if constexpr (MODE == Mode::StateOnly) {
        __syncthreads();
        for (int e = tid; e < D * DV; e += kThreads) gs[(int64_t)(e / DV) * p.DVT + e % DV] = sS[e];
    }

    // Carried-out state, from the workgroup that processes the chain's last tile in scan order
    // (the tile is still in LDS).  Forward: the final state, the last tile's update over its `leff`
    // real positions.  Reverse: lam times the state at position 0, the update over tile 0 (rows
    // past T are zero) -- the gradient of a carried-in forward state.
    if constexpr (kOut) {
        if (p.state_out != nullptr && (DIR == Dir::Forward ? seg == p.nseg - 1 : seg == 0)) {
            __syncthreads();
            const int leff = (int)min((int64_t)TB, T - (DIR == Dir::Forward ? tile_hi - 1 : tile_lo) * TB);
            const float f = DIR == Dir::Forward ? pw(leff) : (end_init && ntiles == 1 ? pw(leff_end - 1) : pw(TB));
            const float scale = DIR == Dir::Forward ? 1.0f : pw(1);
            float *so = p.state_out + (int64_t)chain * D * p.DVT + dv0;
            for (int e = tid; e < D * DV; e += kThreads) {
                const int c = e / DV, n = e % DV;
                float acc = sS[e] * f;
                for (int j = 0; j < leff; ++j)
                    acc = fmaf(sK[j * D + c] * pw(DIR == Dir::Forward ? leff - 1 - j : j), sV[j * DV + n], acc);
                so[(int64_t)c * p.DVT + n] = acc * scale;
            }
        }
    }
}

template <int D, int TB, Dir DIR, Mode MODE>
hipError_t launch_one(const ScanArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)a.chains * a.seg_count * a.nslice;
    hipLaunchKernelGGL((scan_f32_kernel<D, 64, TB, DIR, MODE>), dim3((unsigned)items), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int D, int TB>
hipError_t launch_dm(const ScanArgs &a, Dir dir, Mode mode, hipStream_t s) {
    if (dir == Dir::Forward)
        return mode == Mode::Output ? launch_one<D, TB, Dir::Forward, Mode::Output>(a, s)
                                    : launch_one<D, TB, Dir::Forward, Mode::StateOnly>(a, s);
    return mode == Mode::Output ? launch_one<D, TB, Dir::Reverse, Mode::Output>(a, s)
                                : launch_one<D, TB, Dir::Reverse, Mode::StateOnly>(a, s);
}

template <int D>
hipError_t launch_tb(const ScanArgs &a, int TB, Dir dir, Mode mode, hipStream_t s) {
    if (TB == 16) return launch_dm<D, 16>(a, dir, mode, s);
    if (TB == 32) return launch_dm<D, 32>(a, dir, mode, s);
    return launch_dm<D, 64>(a, dir, mode, s);
}

}  // namespace

bool f32_supported(int D, int DV, int TB) {
    return (D == 64 || D == 128) && DV == 64 && (TB == 16 || TB == 32 || TB == 64);
}

hipError_t launch_scan_f32(const ScanArgs &a, int D, int DV, int TB, Dir dir, Mode mode, hipStream_t s) {
    if (!f32_supported(D, DV, TB)) return hipErrorInvalidValue;
    return D == 64 ? launch_tb<64>(a, TB, dir, mode, s) : launch_tb<128>(a, TB, dir, mode, s);
}

}  // namespace la2
