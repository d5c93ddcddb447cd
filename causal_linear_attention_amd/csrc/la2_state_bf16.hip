// la2_state_bf16.hip -- state-only pass of split chains: each segment's state delta (bf16 in, fp32 out).
//
// When a chain is cut into segments (page "Lightning Attention", lizeman.github.io llm-arch-kb,
// section 2, Step 4 and "Memory footprint": the d x d_v state is the whole hand-over between
// tiles), every segment but one needs the state its predecessors leave behind.  This pass gives
// each segment its own delta, the state it would reach from zero,
//   forward: dS = sum_t lam^(end - t) k_t v_t^T     (end = the segment's last position)
//   reverse: dR = sum_t lam^(t - start) q_t do_t^T  (start = its first position)
// which the segment prefix then chains.  The sum does not depend on how the segment is tiled, so
// this kernel uses its own tile of 64 positions whatever tile the output pass runs with.
//
// Only two operand tiles per step and no outputs: the work per byte is small, and one tile of
// loads in flight per compute unit leaves HBM idle between the request and its data.  So the
// tiles go global -> LDS by direct loads into a ring of kBuf buffers, kBuf - 1 tiles ahead of the
// one being summed, and each step waits only for its own tile (vmcnt counts the younger tiles'
// loads still allowed in flight).  Per tile: S += (w K)^T V on MFMA, fp32 accumulators in
// registers, w the row weights above (applied to a bf16 copy of K in LDS when there is a decay).
#include "la2_bf16_common.h"

namespace la2 {
namespace {

using namespace dev;

constexpr int kTileS = 64;     // positions per tile of this pass
constexpr int kBufMax = 8;     // most tile buffers in the ring (as many as LDS holds, up to this)

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `younger` (0 .. Y) tiles of LPT loads each are still in flight.
template <int LPT, int Y>
__device__ __forceinline__ void wait_tiles(int younger) {
    if constexpr (Y == 0) {
        wait_vm_n<0>();
    } else {
        if (younger >= Y) wait_vm_n<Y * LPT>();
        else wait_tiles<LPT, Y - 1>(younger);
    }
}

template <int D, int DV, Dir DIR, bool DECAY>
__global__ __launch_bounds__(kThreads, 1) void state_bf16_kernel(ScanArgs p) {
    constexpr int TB = kTileS;
    constexpr int TILE = TB * D + TB * DV;   // one buffer: K rows, then V rows (bf16 elements)
    constexpr int oK = 0, oV = TB * D;
    constexpr int KWZ = DECAY ? TB * D : 0;   // decay: K rows weighted by w (bf16)
    constexpr int kFit = (80 * 1024 - KWZ) / TILE;
    constexpr int kBuf = kFit < kBufMax ? kFit : kBufMax;
    constexpr int oKW = kBuf * TILE;
    constexpr int kLds = oKW + KWZ;
    constexpr int NDB = DV / 32, NSB = (D / 32) * NDB;
    constexpr int SPW = NSB > kWaves ? NSB / kWaves : 1;   // 32x32 state blocks per wave
    // direct loads per wave and tile (dma_rows issues RL * NR / 8 / 64 / kWaves per matrix)
    constexpr int LPT = (TB * D / 8 / 64 + TB * DV / 8 / 64) / kWaves;
    static_assert(kBuf >= 3 && kLds * 2 <= 160 * 1024, "LDS");
    static_assert(SPW * kWaves == NSB || (SPW == 1 && NSB <= kWaves), "state blocks");
    __shared__ __attribute__((aligned(16))) u16 smem[kLds];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;

    int item = blockIdx.x;
    if (p.nslice > 1 && gridDim.x % (8 * p.nslice) == 0) {
        // the slices of one segment on one XCD: their k tiles come from one L2
        const int xcd = item & 7, j = item >> 3;
        item = ((j / p.nslice) * 8 + xcd) * p.nslice + j % p.nslice;
    }
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

    const u16 *gb = static_cast<const u16 *>(p.b) + (int64_t)chain * T * D;
    const u16 *gc = static_cast<const u16 *>(p.c) + (int64_t)chain * T * p.DVT + dv0;
    const int sidx = state_index(seg, p.sub, p.nsub, DIR == Dir::Reverse);
    float *gs = p.states + ((int64_t)chain * p.nsub + sidx) * D * p.DVT + dv0;
    const float l2 = DECAY ? log2f(p.decay[chain % p.H]) : 0.0f;

    // Tiles are visited from the far end of the sum's weights: forward from the segment's last tile
    // back, reverse from its first on, so tile `it` has the weights of its rows times lam^(TB it).
    auto tile_of = [&](int it) -> int64_t { return DIR == Dir::Forward ? tile_hi - 1 - it : tile_lo + it; };
    auto issue = [&](u16 *buf, int it) {
        const int64_t t0 = tile_of(it) * TB;
        dma_rows<D, TB>(make_rsrc(gb + t0 * D, (T - t0) * D * 2), buf + oK, D, wave, lane);
        dma_rows<DV, TB>(make_rsrc(gc + t0 * p.DVT, (T - t0) * p.DVT * 2), buf + oV, p.DVT, wave, lane);
    };

    f32x16 sacc[SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[s][r] = 0.0f;
    const bool s_active = wave * SPW < NSB;

#pragma unroll
    for (int it = 0; it < kBuf - 1; ++it)
        if (it < ntiles) issue(smem + it * TILE, it);

    for (int it = 0; it < ntiles; ++it) {
        // this wave's loads of tile `it` have landed once at most the younger tiles' loads are pending
        wait_tiles<LPT, kBuf - 2>(min(ntiles - 1 - it, kBuf - 2));
        lds_barrier();   // ... everyone's; and every wave is done with the tile before it
        // The buffers are distinct and nothing else touches them, which the restrict qualifiers
        // state; without that the compiler makes the fragment reads wait for the loads in flight.
        [&](const u16 *__restrict__ cur, u16 *__restrict__ ahead) __attribute__((always_inline)) {
            if (it + kBuf - 1 < ntiles) issue(ahead, it + kBuf - 1);
            const u16 *sK = cur + oK;
            if constexpr (DECAY) {
                build_kw<D, TB, DIR>(cur + oK, smem + oKW, tid, l2, TB * it);
                lds_barrier();
                sK = smem + oKW;
            }
            if (s_active) {
#pragma unroll
                for (int x = 0; x < TB / 16; ++x)
#pragma unroll
                    for (int s = 0; s < SPW; ++s) {
                        const int sb = wave * SPW + s;
                        sacc[s] = mfma(frag_tr<D, false>(sK, 16 * x, (sb / NDB) * 32, lane),
                                       frag_tr<DV, false>(cur + oV, 16 * x, (sb % NDB) * 32, lane), sacc[s]);
                    }
            }
        }(smem + (it % kBuf) * TILE, smem + ((it + kBuf - 1) % kBuf) * TILE);
        // the next step's barrier also keeps the weighted copy until every wave has read it
    }

    if (s_active) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int sb = wave * SPW + s, kb = sb / NDB, nb = sb % NDB;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                gs[(int64_t)d * p.DVT + nb * 32 + col] = sacc[s][r];
            }
        }
    }
}

template <int D, int DV, Dir DIR>
hipError_t launch_dv(const ScanArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)a.chains * a.seg_count * a.nslice;
    if (a.decay)
        hipLaunchKernelGGL((state_bf16_kernel<D, DV, DIR, true>), dim3((unsigned)items), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((state_bf16_kernel<D, DV, DIR, false>), dim3((unsigned)items), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_d(const ScanArgs &a, Dir dir, hipStream_t s) {
    return dir == Dir::Forward ? launch_dv<D, DV, Dir::Forward>(a, s) : launch_dv<D, DV, Dir::Reverse>(a, s);
}

}  // namespace

hipError_t launch_state_bf16(const ScanArgs &args, int D, int DV, int TB, Dir dir, hipStream_t s) {
    if (!(D == 64 || D == 128) || !(DV == 64 || DV == 128) || TB % kTileS != 0 || args.states == nullptr)
        return hipErrorInvalidValue;
    // segments are given in tiles of the output pass; this pass counts its own
    ScanArgs a = args;
    a.seg_tiles = args.seg_tiles * (TB / kTileS);
    if (D == 64) return DV == 64 ? launch_d<64, 64>(a, dir, s) : launch_d<64, 128>(a, dir, s);
    return DV == 64 ? launch_d<128, 64>(a, dir, s) : launch_d<128, 128>(a, dir, s);
}

}  // namespace la2
