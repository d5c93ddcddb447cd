// la2_fwd1_bf16.hip -- the forward output scan without decay at d = d_v = 128 in bf16, as producer and
// consumer waves over 64-position tiles.
//
// Page "Lightning Attention" (lizeman.github.io llm-arch-kb), section 2, Steps 1-4: per tile b of
// 64 positions (local rows t = outputs, s = sources)
//   O_b = mask(Q_b K_b^T) V_b + Q_b S_{b-1}    (intra: sources s <= t; inter: the state before the tile)
//   S_b = S_{b-1} + K_b^T V_b                  (the state update on the unmasked tile)
// and with a per-head decay lam (the recurrence S_t = lam S_{t-1} + k_t v_t^T):
//   O_b[t] = sum_{s<=t} lam^(t-s) (q_t . k_s) v_s + lam^(t+1) q_t S_{b-1},
//   S_b = lam^64 S_{b-1} + sum_j lam^(63-j) k_j v_j^T.
// and, with a key/value pair of roles (b, c) and a query role a, the same scan serves the dQ pass of
// the two-pass backward and the scan U of the normalized backward (its state read transposed); the
// latter, with (a, b) = (do, v), also writes each row's do_t . (the prefix sum of v through t), by
// the normalized form's denominator machinery below without the division.
//
// Workgroup of eight waves, two per SIMD, in two roles (the layout of the one-pass backward):
//   consumers (waves 0-3, c = 2rb + ch): columns 64ch..64ch+63 of the output rows in block rb;
//   producers (waves 4-7, p): the fp32 state rows 32p..32p+31 (all 128 columns) in registers,
//     updated with the tile's K^T V and published as a bf16 copy S^T in LDS.
// The state update of tile b overlaps the consumers' products of tile b on every SIMD; S_b's copy
// replaces S_{b-1}'s only after barrier Y, when every consumer is done reading it.  The next tile's
// q, k and v go global -> LDS by direct loads into the second of two tile buffers, issued at the top
// of the tile, so they have the whole tile to land.  Two barriers per tile: Y and X (the next tile
// and S_b's copy in LDS).  LDS: 2 x (q, k, v) 96 KiB, S^T 32 KiB, output staging 4 x 4 KiB.
//
// The normalized form (page "Lightning Attention", section 1: numerator over denominator, with a
// feature map phi on q and k): o_t = S_t^T phi(q_t) / (phi(q_t) . z_t), z_t = sum_{s<=t} phi(k_s).
// phi is applied to the q and k tiles on their way into LDS (rows past the sequence stay zero), so the
// numerator is the plain scan on phi(q), phi(k) rounded to bf16.  With elu + 1, k goes through the
// producers' registers: k of tile b + 1 is loaded at the top of tile b - 1 and, transformed, written to
// LDS at the top of tile b, beside the consumers' products of tile b; q arrives by direct loads, and
// each wave transforms the chunks its own loads filled after barrier Y, once they have landed (so only
// half the transform waits between barriers Y and X).  The denominator comes from the same rounded
// values: its intra-tile part is the sum of each output row's kept fp32 scores, its inter part the product of the
// row with z before the tile, which the producers keep in fp32 from their K^T operands (column sums of
// phi(K)) and publish beside S^T as two bf16 rows (z rounded, and the remainder rounded) of an
// otherwise zero [32][128] tile, so that the consumers take it with 8 more MFMAs beside their inter
// product.  Each output row is divided in fp32 before it is rounded.
#include "la2_tile64_bf16.h"

namespace la2 {
namespace {

using namespace dev;
using namespace t64;

constexpr int kTF = 512;                      // threads: 4 consumers, then 4 producers
constexpr int oQF = 0, oKF = kTile1, oVF = 2 * kTile1;   // within a tile buffer
constexpr int kBufF = 3 * kTile1;             // one buffer of the three input tiles
constexpr int oSTF = 2 * kBufF;               // S^T [d_v][d] bf16
constexpr int oOSF = oSTF + D1 * D1;          // per-consumer output staging, 32 x 64
constexpr int kOSF = 32 * 64;
constexpr int oZF = oOSF + 4 * kOSF;          // the normalized form: z before the tile, [32][128] bf16
constexpr int kLdsF = oZF + 32 * D1;
static_assert(kLdsF * 2 <= 160 * 1024, "LDS");
static_assert(kWaves == 8, "the direct loads split a tile over eight waves");

// The 64-position tiles of one (chain, segment), first to last.
struct WalkF {
    int64_t T, t_lo, base;
    int ntiles;
    __device__ int64_t t0(int it) const { return t_lo + (int64_t)it * TB1; }
};

__device__ __forceinline__ WalkF walk_of(const Fwd1Args &p, int chain, int seg) {
    WalkF w;
    w.T = p.T;
    w.t_lo = (int64_t)seg * p.seg_len;
    const int64_t t_hi = min(p.T, w.t_lo + p.seg_len);
    w.ntiles = (int)((t_hi - w.t_lo + TB1 - 1) / TB1);
    w.base = (int64_t)chain * p.T * D1;
    return w;
}

// The tile starting at t0 of q, k and v into one LDS buffer (rows past T arrive as zeros).
__device__ __forceinline__ void dma_tile_f(u16 *buf, const u16 *gq, const u16 *gk, const u16 *gv, int64_t t0,
                                           int64_t T, int wave, int lane) {
    const int64_t bytes = (T - t0) * D1 * 2;
    dma_rows<D1, TB1>(make_rsrc(gq + t0 * D1, bytes), buf + oQF, D1, wave, lane);
    dma_rows<D1, TB1>(make_rsrc(gk + t0 * D1, bytes), buf + oKF, D1, wave, lane);
    dma_rows<D1, TB1>(make_rsrc(gv + t0 * D1, bytes), buf + oVF, D1, wave, lane);
}

// Only the q and v tiles of the tile starting at t0 (the elu + 1 form, whose k goes through the
// producers' registers).
__device__ __forceinline__ void dma_qv_f(u16 *buf, const u16 *gq, const u16 *gv, int64_t t0, int64_t T, int wave,
                                         int lane) {
    const int64_t bytes = (T - t0) * D1 * 2;
    dma_rows<D1, TB1>(make_rsrc(gq + t0 * D1, bytes), buf + oQF, D1, wave, lane);
    dma_rows<D1, TB1>(make_rsrc(gv + t0 * D1, bytes), buf + oVF, D1, wave, lane);
}

// elu + 1: x + 1 above zero, e^x at or below.  e^x clamped to [0, 1] (the clamp output modifier of
// the exp instruction) is e^min(x, 0), and e^x >= x + 1 everywhere, so the larger of x + 1 and the
// clamped exponential is elu + 1 without a compare and select; the NaN-propagating maximum keeps a
// NaN input NaN.
__device__ __forceinline__ float elu1(float x) {
    const float e = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * 1.44269502f), 0.0f, 1.0f);
    return __builtin_elementwise_maximum(x + 1.0f, e);
}

// The k chunks of one tile that producer pw carries in registers (the elu + 1 form): chunks
// c = 64 i + lane, i = pw + 4 s, of each tile, placed where dma_rows would put them.
constexpr int kKC = kTile1 / 8 / 256;   // chunks per lane (4)
struct KRegs {
    u32x4 k[kKC];
};

__device__ __forceinline__ void load_k(KRegs &r, const u16 *gk, int64_t t0, int64_t T, int pw, int lane) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(gk + t0 * D1, (T - t0) * D1 * 2);
#pragma unroll
    for (int s = 0; s < kKC; ++s) {
        const int c = 64 * (pw + 4 * s) + lane, row = c / (D1 / 8), lc = (c % (D1 / 8)) ^ swz<D1>(row);
        r.k[s] = bload(rk, (row * D1 + lc * 8) * 2);
    }
}

// phi = elu + 1 on the loaded chunks (rows past the sequence arrive as zeros and stay zero) into the
// k tile of `buf`, and to pk where asked for.
__device__ __forceinline__ void put_k(KRegs &r, u16 *buf, const Fwd1Args &p, int64_t base, int64_t t0, int64_t T,
                                      int pw, int lane) {
    u16 *gpk = p.pk ? static_cast<u16 *>(p.pk) + base + t0 * D1 : nullptr;
#pragma unroll
    for (int s = 0; s < kKC; ++s) {
        const int c = 64 * (pw + 4 * s) + lane, row = c / (D1 / 8), lc = (c % (D1 / 8)) ^ swz<D1>(row);
        const bool real = t0 + row < T;
        u32x4 x = r.k[s];
        if (real) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = pack_bf16(elu1(__builtin_bit_cast(float, x[j] << 16)),
                                 elu1(__builtin_bit_cast(float, x[j] & 0xffff0000u)));
        }
        *reinterpret_cast<u32x4 *>(buf + oKF + 8 * c) = x;
        if (gpk && real) bstore16(make_rsrc(gpk, (T - t0) * D1 * 2), (row * D1 + lc * 8) * 2, x);
    }
}

// phi = elu + 1 on the chunks of the q and k tiles in `buf` that dma_tile_f's share `share` filled
// (rows past the sequence stay zero), and the transformed chunks to pq, pk where asked for.  Only the
// wave that issued those loads may call it, after waiting for them: no other wave touches the chunks.
template <bool WITH_K = true>
__device__ __forceinline__ void phi_share(u16 *buf, const Fwd1Args &p, int64_t base, int64_t t0, int64_t T,
                                          int share, int lane) {
    const int64_t bytes = (T - t0) * D1 * 2;
    u16 *gpq = p.pq ? static_cast<u16 *>(p.pq) + base + t0 * D1 : nullptr;
    u16 *gpk = p.pk ? static_cast<u16 *>(p.pk) + base + t0 * D1 : nullptr;
#pragma unroll
    for (int s = 0; s < kTile1 / (512 * kWaves); ++s) {
        const int i = share + kWaves * s, c = 64 * i + lane, row = c / (D1 / 8);
        const int lc = (c % (D1 / 8)) ^ swz<D1>(row);
        if (t0 + row >= T) continue;
#pragma unroll
        for (int tns = 0; tns < (WITH_K ? 2 : 1); ++tns) {
            u16 *l = buf + (tns ? oKF : oQF) + 8 * c;
            u32x4 x = *reinterpret_cast<const u32x4 *>(l);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = pack_bf16(elu1(__builtin_bit_cast(float, x[j] << 16)),
                                 elu1(__builtin_bit_cast(float, x[j] & 0xffff0000u)));
            *reinterpret_cast<u32x4 *>(l) = x;
            u16 *g = tns ? gpk : gpq;
            if (g) bstore16(make_rsrc(g, bytes), (row * D1 + lc * 8) * 2, x);
        }
    }
}

__device__ __forceinline__ float chain_l2(const Fwd1Args &p, int chain) {
    return p.decay != nullptr ? log2f(p.decay[chain % p.H]) : 0.0f;
}

// The value tile as kappa = phi(x) - m (NM = 3: identity, 4: elu + 1) on the chunks of `buf` that
// dma_tile_f's share `share` filled, with m[8 lc + e] in mv[e] (lc the lane's column block, the same
// for both of its chunks; rows past the sequence stay zero): the scan of the normalized backward's bf16
// dq, whose value role is the centered feature map of the keys.  Only the wave that issued those loads
// may call it, after waiting for them.
template <int NM>
__device__ __forceinline__ void center_share(u16 *buf, int64_t t0, int64_t T, int share, int lane,
                                             const float (&mv)[8]) {
#pragma unroll
    for (int s = 0; s < kTile1 / (512 * kWaves); ++s) {
        const int i = share + kWaves * s, c = 64 * i + lane, row = c / (D1 / 8);
        if (t0 + row >= T) continue;
        u16 *l = buf + oVF + 8 * c;
        u32x4 x = *reinterpret_cast<const u32x4 *>(l);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float lo = __builtin_bit_cast(float, x[j] << 16), hi = __builtin_bit_cast(float, x[j] & 0xffff0000u);
            if constexpr (NM == 4) {
                lo = elu1(lo);
                hi = elu1(hi);
            }
            x[j] = pack_bf16(lo - mv[2 * j], hi - mv[2 * j + 1]);
        }
        *reinterpret_cast<u32x4 *>(l) = x;
    }
}

// m[8 lc + e] for the column block lc of the lane's chunks in share `share`: the chain's mean of the
// feature map of the keys, from the sums over the segments of msum_seg positions.
__device__ __forceinline__ void center_means(const Fwd1Args &p, int chain, int share, int lane, float (&mv)[8]) {
    const int c0 = 64 * share + lane, row0 = c0 / (D1 / 8), lc = (c0 % (D1 / 8)) ^ swz<D1>(row0);
    const int64_t nms = (p.T + p.msum_seg - 1) / p.msum_seg;
    const float *ms = p.msum + (int64_t)chain * nms * D1 + lc * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] = 0.0f;
    for (int64_t j = 0; j < nms; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) mv[e] += ms[j * D1 + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] /= (float)p.T;
}

// Producer p: state rows 32p..32p+31 of S (d x d_v), four 32 x 32 blocks (column blocks jb).
template <int NM, bool DEC>
__device__ __forceinline__ void producer_f(const Fwd1Args &p, u16 *smem, int chain, int seg, int pw, int lane) {
    const WalkF w = walk_of(p, chain, seg);
    const int wave = 4 + pw, h = lane >> 5, col = lane & 31;
    // per-lane LDS offsets: transposed reads of K's column block pw and of V's four column blocks, and
    // where accumulator entries 4q..4q+3 (state rows 32pw + 8q + 4h..) land in a row of S^T
    int trk[2], trv[4][2], pwq[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        trk[half] = tr_off(lane, 0, half, pw);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) trv[jb][half] = tr_off(lane, 0, half, jb);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) pwq[q] = nat_off<D1>(col, 4 * pw + q) + 4 * h;
    const u16 *gq = static_cast<const u16 *>(p.q) + w.base, *gk = static_cast<const u16 *>(p.k) + w.base;
    const u16 *gv = static_cast<const u16 *>(p.v) + w.base;
    const bool last_seg = seg == p.nseg - 1;
    const bool final_state = last_seg && p.state_out != nullptr;

    // the state the segment starts from: zero, or the segment's entry of the start states ([D][DV], or
    // [DV][D] when read transposed)
    f32x16 sacc[4];
    const float *g = seg > 0 && p.states != nullptr
                         ? p.states + ((int64_t)chain * p.nsub + state_index(seg, p.sub, p.nsub, false)) * D1 * D1
                         : nullptr;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = pw * 32 + 8 * (r >> 2) + 4 * h + (r & 3), j = jb * 32 + col;
            sacc[jb][r] = g != nullptr ? g[p.states_t ? (int64_t)j * D1 + i : (int64_t)i * D1 + j] : 0.0f;
        }
    // the normalized form: this lane's half (positions 8h.. of every 16) of the prefix sum of phi(k) in
    // state row 32pw + col; and the whole sum where the last segment sum was written
    float zacc = 0.0f, zmark = 0.0f;
    auto z_whole = [&]() {
        const unsigned int zu = __builtin_bit_cast(unsigned int, zacc);
        const auto r = __builtin_amdgcn_permlane32_swap(zu, zu, false, false);
        return __builtin_bit_cast(float, (unsigned int)r[0]) + __builtin_bit_cast(float, (unsigned int)r[1]);
    };
    constexpr bool NRM = NM == 1 || NM == 2;   // the normalized forward (its segment sums of phi(k))
    constexpr bool ZS = NM >= 1;               // z and the rows' sums (every normalized instance)
    const bool sums = NRM && p.msum != nullptr;
    float mv[8];
    if constexpr (NM >= 3) center_means(p, chain, wave, lane, mv);
    // a decay: lam^64 per tile on the state, and lam^(63 - j) on the K^T operand's position j =
    // 16x + 8h + e (element e of the fragment of step x)
    float wk[DEC ? TB1 / 16 : 1][8], lam64 = 1.0f;
    const float l2 = DEC ? chain_l2(p, chain) : 0.0f;
    if constexpr (DEC) {
        lam64 = exp2f(64.0f * l2);
#pragma unroll
        for (int x = 0; x < TB1 / 16; ++x)
#pragma unroll
            for (int e = 0; e < 8; ++e) wk[x][e] = exp2f(l2 * (float)(TB1 - 1 - (16 * x + 8 * h + e)));
    }
    // the bf16 copy S^T ([d_v][d]): accumulator entries 4q..4q+3 are four consecutive d of one d_v row;
    // and z (fp32), whole in every lane after adding the partner lane's half
    auto write_state = [&]() {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 v = {pack_bf16(sacc[jb][4 * q], sacc[jb][4 * q + 1]),
                                 pack_bf16(sacc[jb][4 * q + 2], sacc[jb][4 * q + 3])};
                lds_write8(smem + oSTF, jb * 32 * D1 + pwq[q], v);
            }
        if constexpr (ZS) {
            const float z = z_whole();
            // z of column 32pw + col in row 0 (rounded to bf16) and row 1 (the remainder) of the z tile;
            // lanes h = 0 write row 0, h = 1 row 1
            const u16 zh = __builtin_bit_cast(u16, (__bf16)z);
            const float zr = z - __builtin_bit_cast(float, (unsigned int)zh << 16);
            const int dcol = pw * 32 + col;
            smem[oZF + nat_off<D1>(h, dcol >> 3) + (dcol & 7)] = h == 0 ? zh : __builtin_bit_cast(u16, (__bf16)zr);
        }
    };
    dma_tile_f(smem, gq, gk, gv, w.t0(0), w.T, wave, lane);
    if constexpr (ZS) {
        // the z tile's zero rows 2..31 (rows 0 and 1 come with every copy of the state)
        const u32x4 zz = {0u, 0u, 0u, 0u};
        for (int i = (wave - 4) * 64 + lane; i < 30 * D1 / 8; i += 256)
            *reinterpret_cast<u32x4 *>(smem + oZF + 2 * D1 + 8 * i) = zz;
    }
    write_state();
    // the elu + 1 form: k of tile it + 1 waits in registers during tile it - 1 and goes to LDS,
    // transformed, at the top of tile it, beside the consumers' products; q is transformed after barrier Y
    KRegs kr;
    if (NM == 2 && w.ntiles > 1) load_k(kr, gk, w.t0(1), w.T, pw, lane);
    wait_vm();
    if constexpr (NM == 2) phi_share(smem, p, w.base, w.t0(0), w.T, wave, lane);
    if constexpr (NM >= 3) center_share<NM>(smem, w.t0(0), w.T, wave, lane, mv);
    lds_barrier();   // X: the first tile and S^T
    for (int it = 0; it < w.ntiles; ++it) {
        const bool more = it + 1 < w.ntiles;
        // the two tile buffers are distinct and nothing else touches them, which the restrict
        // qualifiers state: without that the compiler makes the transposed fragment reads of this
        // tile wait for the next tile's direct loads
        [&](const u16 *__restrict__ cur, u16 *__restrict__ nxt) __attribute__((always_inline)) {
            if constexpr (NM == 2) {
                if (more) {
                    dma_qv_f(nxt, gq, gv, w.t0(it + 1), w.T, wave, lane);
                    put_k(kr, nxt, p, w.base, w.t0(it + 1), w.T, pw, lane);
                    if (it + 2 < w.ntiles) load_k(kr, gk, w.t0(it + 2), w.T, pw, lane);
                }
            } else if (more) {
                dma_tile_f(nxt, gq, gk, gv, w.t0(it + 1), w.T, wave, lane);
            }
            // S += K^T V over the tile's 64 positions (the last tile's update only for the final state or the
            // segment sums of phi(k))
            if (more || final_state || sums) {
                const u16 *sK = cur + oKF, *sV = cur + oVF;
                if (DEC && !more) {
                    // the final state's tile: its n real rows, lam^n on the state and lam^(n - 1 - j) on row j
                    const int n = (int)min((int64_t)TB1, w.T - w.t0(it));
                    lam64 = exp2f(l2 * (float)n);
    #pragma unroll
                    for (int x = 0; x < TB1 / 16; ++x)
    #pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 16 * x + 8 * h + e;
                            wk[x][e] = j < n ? exp2f(l2 * (float)(n - 1 - j)) : 0.0f;
                        }
                }
                if constexpr (DEC) {
    #pragma unroll
                    for (int jb = 0; jb < 4; ++jb)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[jb][r] *= lam64;
                }
    #pragma unroll
                for (int x = 0; x < TB1 / 16; ++x) {
                    bf16x8 fa = rd_tr(sK, 16 * x, trk);
                    if constexpr (DEC) {
                        u32x4 u = __builtin_bit_cast(u32x4, fa);
    #pragma unroll
                        for (int j = 0; j < 4; ++j)
                            u[j] = pack_bf16(__builtin_bit_cast(float, u[j] << 16) * wk[x][2 * j],
                                             __builtin_bit_cast(float, u[j] & 0xffff0000u) * wk[x][2 * j + 1]);
                        fa = __builtin_bit_cast(bf16x8, u);
                    }
                    bf16x8 fc[4];
    #pragma unroll
                    for (int jb = 0; jb < 4; ++jb) fc[jb] = rd_tr(sV, 16 * x, trv[jb]);
    #pragma unroll
                    for (int jb = 0; jb < 4; ++jb) sacc[jb] = mfma(fa, fc[jb], sacc[jb]);
                    if constexpr (ZS) {
                        // fa: state row 32pw + col of K^T at positions 16x + 8h .. 16x + 8h + 7
                        const u32x4 u = __builtin_bit_cast(u32x4, fa);
    #pragma unroll
                        for (int j = 0; j < 4; ++j)
                            zacc += __builtin_bit_cast(float, u[j] << 16) + __builtin_bit_cast(float, u[j] & 0xffff0000u);
                    }
                }
            }
            if constexpr (NRM) {
                // the sum of phi(k) over a segment of msum_seg positions, written at its last tile
                const int64_t t_end = w.t0(it) + TB1;
                if (sums && (!more || t_end % p.msum_seg == 0)) {
                    const float z = z_whole();
                    const int64_t nms = (w.T + p.msum_seg - 1) / p.msum_seg, ms = (t_end - 1) / p.msum_seg;
                    if (h == 0) p.msum[((int64_t)chain * nms + ms) * D1 + pw * 32 + col] = z - zmark;
                    zmark = z;
                }
            }
            lds_barrier();   // Y: every consumer is done with S_{b-1}^T (and z before the tile)
            if (more) write_state();
            wait_vm();
            if (NM == 2 && more) phi_share<false>(nxt, p, w.base, w.t0(it + 1), w.T, wave, lane);
            if (NM >= 3 && more) center_share<NM>(nxt, w.t0(it + 1), w.T, wave, lane, mv);
            lds_barrier();   // X: the next tile and S_b^T
        }(smem + (it & 1) * kBufF, smem + ((it + 1) & 1) * kBufF);
    }
    if (final_state) {
        float *so = p.state_out + (int64_t)chain * D1 * D1;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = pw * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                so[(int64_t)i * D1 + jb * 32 + col] = sacc[jb][r];
            }
    }
}

// Consumer c = 2rb + ch: the output unit of row block rb, columns 64ch..64ch+63, staged in the wave's
// own 4 KiB of LDS and stored as whole 128-byte row pieces at the top of the next tile.
template <int NM, bool DEC>
__device__ __forceinline__ void consumer_f(const Fwd1Args &p, u16 *smem, int chain, int seg, int c, int lane) {
    const WalkF w = walk_of(p, chain, seg);
    const int rb = c >> 1, ch = c & 1;
    const LaneOff L = lane_offsets(lane, ch);
    DecayW dwt = {};   // read only with a decay
    if constexpr (DEC) dwt = decay_weights<true>(chain_l2(p, chain), rb, lane);
    const u16 *gq = static_cast<const u16 *>(p.q) + w.base, *gk = static_cast<const u16 *>(p.k) + w.base;
    const u16 *gv = static_cast<const u16 *>(p.v) + w.base;
    u16 *gy = static_cast<u16 *>(p.y) + w.base;
    u16 *ob = smem + oOSF + c * kOSF;
    auto stage = [&](const f32x16 (&acc)[2]) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 v = {pack_bf16(acc[n][4 * q], acc[n][4 * q + 1]),
                                 pack_bf16(acc[n][4 * q + 2], acc[n][4 * q + 3])};
                lds_write8(ob, L.po[n][q], v);
            }
    };
    auto store = [&](int64_t t0) {
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(gy + t0 * D1, (w.T - t0) * D1 * 2);
        u32x4 v[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int qd = lane + 64 * s2, row = qd / 8, chk = qd % 8;
            v[s2] = *reinterpret_cast<const u32x4 *>(ob + row * 64 + ((chk ^ ((row >> 1) & 7)) << 3));
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int qd = lane + 64 * s2, row = qd / 8, chk = qd % 8;
            bstore16(ry, ((rb * 32 + row) * D1 + ch * 64 + chk * 8) * 2, v[s2]);
        }
    };

    dma_tile_f(smem, gq, gk, gv, w.t0(0), w.T, c, lane);
    wait_vm();
    float mv[8];
    if constexpr (NM >= 3) center_means(p, chain, c, lane, mv);
    if constexpr (NM == 2) phi_share(smem, p, w.base, w.t0(0), w.T, c, lane);
    if constexpr (NM >= 3) center_share<NM>(smem, w.t0(0), w.T, c, lane, mv);
    lds_barrier();   // X: the first tile and S^T
    for (int it = 0; it < w.ntiles; ++it) {
        const bool more = it + 1 < w.ntiles;
        // the two tile buffers are distinct and nothing else touches them, which the restrict
        // qualifiers state: without that the compiler makes the transposed fragment reads of this
        // tile wait for the next tile's direct loads
        [&](const u16 *__restrict__ cur, u16 *__restrict__ nxt) __attribute__((always_inline)) {
            if (more) {
                if constexpr (NM == 2)
                    dma_qv_f(nxt, gq, gv, w.t0(it + 1), w.T, c, lane);
                else
                    dma_tile_f(nxt, gq, gk, gv, w.t0(it + 1), w.T, c, lane);
            }
            if (it > 0) store(w.t0(it - 1));
            {
                f32x16 oacc[2];
                if constexpr (NM >= 1) {
                    float dpart;
                    unit_products<true, true, true, false>(oacc, cur + oQF, cur + oKF, cur + oVF, smem + oSTF, rb, ch,
                                                           lane, L, &dpart, smem + oZF, dwt);
                    const unsigned int du = __builtin_bit_cast(unsigned int, dpart);
                    const auto r = __builtin_amdgcn_permlane32_swap(du, du, false, false);
                    const float den =
                        __builtin_bit_cast(float, (unsigned int)r[0]) + __builtin_bit_cast(float, (unsigned int)r[1]);
                    if constexpr (NM <= 2) {   // the scans U are not divided
                        const float inv = 1.0f / den;
#pragma unroll
                        for (int n = 0; n < 2; ++n)
#pragma unroll
                            for (int e = 0; e < 16; ++e) oacc[n][e] *= inv;
                    }
                    const int64_t t = w.t0(it) + rb * 32 + (lane & 31);
                    if (p.den != nullptr && ch == 0 && lane < 32 && t < w.T) p.den[(int64_t)chain * w.T + t] = den;
                } else {
                    unit_products<true, true, false, DEC>(oacc, cur + oQF, cur + oKF, cur + oVF, smem + oSTF, rb, ch,
                                                          lane, L, nullptr, nullptr, dwt);
                }
                stage(oacc);
            }
            lds_barrier();   // Y
            wait_vm();
            if (NM == 2 && more) phi_share<false>(nxt, p, w.base, w.t0(it + 1), w.T, c, lane);
            if (NM >= 3 && more) center_share<NM>(nxt, w.t0(it + 1), w.T, c, lane, mv);
            lds_barrier();   // X
        }(smem + (it & 1) * kBufF, smem + ((it + 1) & 1) * kBufF);
    }
    store(w.t0(w.ntiles - 1));
}

template <int NM, bool DEC>
__global__ __launch_bounds__(kTF, 1) void fwd1_bf16_kernel(Fwd1Args p) {
    __shared__ __attribute__((aligned(16))) u16 smem[kLdsF];
    // the wave index as a scalar: every branch on a wave's role is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int seg = blockIdx.x % p.nseg;
    const int chain = blockIdx.x / p.nseg;
    if ((int64_t)seg * p.seg_len >= p.T) return;
    if (wave < 4)
        consumer_f<NM, DEC>(p, smem, chain, seg, wave, lane);
    else
        producer_f<NM, DEC>(p, smem, chain, seg, wave - 4, lane);
}

}  // namespace

hipError_t launch_fwd1_bf16(const Fwd1Args &a, hipStream_t s) {
    if (a.seg_len <= 0 || a.seg_len % TB1 != 0 || a.norm < 0 || a.norm > 4) return hipErrorInvalidValue;
    if (a.msum != nullptr && (a.norm == 0 || a.msum_seg <= 0 || a.msum_seg % TB1 != 0)) return hipErrorInvalidValue;
    // the centered value tile needs the segment sums of the feature map of the keys
    if (a.norm >= 3 && a.msum == nullptr) return hipErrorInvalidValue;
    // the normalized form keeps z per chain from zero: unsplit chains only
    if (a.norm != 0 && (a.nseg != 1 || a.states != nullptr || a.state_out != nullptr)) return hipErrorInvalidValue;
    // a decay: the plain scan only
    if (a.decay != nullptr && (a.norm != 0 || a.H <= 0)) return hipErrorInvalidValue;
    const unsigned items = (unsigned)((int64_t)a.chains * a.nseg);
    if (a.decay != nullptr) {
        hipLaunchKernelGGL((fwd1_bf16_kernel<0, true>), dim3(items), dim3(kTF), 0, s, a);
        return hipGetLastError();
    }
    switch (a.norm) {
        case 0: hipLaunchKernelGGL((fwd1_bf16_kernel<0, false>), dim3(items), dim3(kTF), 0, s, a); break;
        case 1: hipLaunchKernelGGL((fwd1_bf16_kernel<1, false>), dim3(items), dim3(kTF), 0, s, a); break;
        case 2: hipLaunchKernelGGL((fwd1_bf16_kernel<2, false>), dim3(items), dim3(kTF), 0, s, a); break;
        case 3: hipLaunchKernelGGL((fwd1_bf16_kernel<3, false>), dim3(items), dim3(kTF), 0, s, a); break;
        default: hipLaunchKernelGGL((fwd1_bf16_kernel<4, false>), dim3(items), dim3(kTF), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace la2
