// la2_bwd1_bf16.hip -- the whole backward pass without decay (lam = 1) in one reverse walk:
// dQ, dK and dV of one (chain, segment) from a single read of q, k, v and dO (bf16, d = d_v = 128).
//
// The backward of the prefix-sum recurrence of page "Lightning Attention" (lizeman.github.io
// llm-arch-kb, section 1) is, with S_t = sum_{s<=t} k_s v_s^T and R_t = sum_{s>=t} q_s do_s^T,
//   dq_t = S_t do_t,   dk_t = R_t v_t,   dv_t = R_t^T k_t,
// and tiled as in section 2, Steps 1-4, per tile b of TB positions (local rows i = outputs):
//   dV_b = mask^T(Q_b K_b^T)^T dO_b + K_b R_{b+1}          (intra: sources t >= s)
//   dK_b = mask^T(dO_b V_b^T)^T Q_b + V_b R_{b+1}^T
//   dQ_b = mask(dO_b V_b^T) K_b + dO_b S_{b-1}^T             (intra: sources s <= t)
//   R_b  = R_{b+1} + Q_b^T dO_b,   S_{b-1} = S_b - K_b^T V_b.
// The walk goes from the segment's last tile to its first, carrying R forward as the dK/dV pass does
// and carrying S backwards from the state at the segment's end: without decay the forward state of
// the tile before is the state after it minus the tile's own K^T V, a subtraction in fp32 whose error
// stays at the rounding of |S|.  (With a decay lam < 1 undoing a tile would divide by lam^TB, which
// amplifies every rounding; decayed chains keep the two-pass backward.)  Reading each input once for
// all three gradients moves 7 tensors per token instead of the 10 of a dQ pass plus a dK/dV pass.
//
// Workgroup of eight waves, two per SIMD, 64-position tiles (two 32-row blocks), in two roles:
//   consumers (waves 0-3, c = 2rb + ch): columns 64ch..64ch+63 of dV, dK and dQ for row block rb
//     (row block 0 has two source blocks for dV and dK and one for dQ, row block 1 the reverse);
//   producers (waves 4-7, p = 4 + 2j + ch): the state blocks with rows kb in {2ch, 2ch + 1} (all four
//     column blocks) of R (j = 0) or S (j = 1) and their bf16 copies in LDS.
// Each SIMD runs one wave of each role, so the state updates and state copies overlap the gradient
// products instead of following them.  Every wave loads an eighth of the next tile into registers
// early in the tile and writes it to LDS once the tile's inputs are consumed.  LDS holds the four input tiles, R^T and S^T in
// bf16 (MFMA operands of the inter-tile products) and 8 KiB of output staging per consumer: 160 KiB.
// Per tile, three workgroup barriers: Y (S^T of the state before the tile is complete, dV and dK are
// done with R^T), Z (every input of the tile is consumed) and X (the next tile and R^T are in LDS).
//
// The same kernel without dQ and S (ONE = false) is the dK/dV pass of the two-pass backward, with an
// optional per-head decay lam (the recurrence R_t = lam R_{t+1} + q_t do_t^T; R here is the state after
// the tile, at its last position + 1):
//   dV_b[t] = sum_{s>=t} lam^(s-t) (q_s . k_t) do_s + lam^(64-t) k_t R_{b+1},   likewise dK_b with
//   (do, v, q);   R_b = lam^64 R_{b+1} + sum_j lam^j q_j do_j^T.
// The S producers then only stage tiles.
//
// With the gradient of the normalized form's denominators (NK; page "Lightning Attention", section 1:
// o_t = n_t / den_t, den_t = phi(q_t) . z_t), run on (phi(q), phi(k), v, dn) with dn_t = do_t / den_t
// (formed here: each do row is scaled by 1 / den_t in fp32 and rounded on its way into LDS) and given
// dden_t = -(do_t . o_t) / den_t, the walk forms the whole gradient with respect to k:
//   d phi(k_s) = sum_{t>=s} (dn_t . v_s + dden_t) phi(q_t),   dk_s = d phi(k_s) (.) phi'(k_s),
// the score of every pair (t, s) taking dden_t on top, the later tiles' part y_{b+1} = sum over them of
// dden_t phi(q_t) (a d-vector the R producers carry beside R), and phi'(k) = min(phi(k), 1) for
// elu + 1 (1 for the identity), from the phi(k) tile; dk is rounded once.  S^T's LDS, unused without
// dQ, holds the tile's dden and y.
#include "la2_tile64_bf16.h"

namespace la2 {
namespace {

using namespace dev;
using namespace t64;

constexpr int kW1 = 8;               // waves: 4 consumers, then 4 producers
constexpr int kT1 = 64 * kW1;        // threads
constexpr int oQ1 = 0, oK1 = kTile1, oV1 = 2 * kTile1, oO1 = 3 * kTile1;   // q, k, v, dO tiles
constexpr int oRT1 = 4 * kTile1;                                           // R^T [d_v][d] bf16
constexpr int oST1 = oRT1 + D1 * D1;                                       // S^T [d_v][d] bf16
constexpr int oOS1 = oST1 + D1 * D1;                                       // per-consumer output staging
constexpr int oDD1 = oST1, oY1 = oST1 + 2 * TB1;   // NK (no S^T): the tile's dden, y (fp32, 64 and 128)
constexpr int kOS1 = 2 * 32 * 64;                                          //   (two units of 32 x 64)
constexpr int kLds1 = oOS1 + 4 * kOS1;
constexpr int NCH1 = kTile1 / 8 / kT1;   // 16-byte chunks per thread and tile (2)
static_assert(kLds1 * 2 <= 160 * 1024, "LDS");


enum class Unit { DV, DK, DQ };

struct Staged1 {
    u32x4 q[NCH1], k[NCH1], v[NCH1], o[NCH1];
    float den[NCH1];   // DS: the denominators of the dO chunks' rows
};

// DS: the dO role is do, its rows divided by den (the chain's [T] denominators) when staged.
template <bool DS = false>
__device__ __forceinline__ void load_tile1(Staged1 &r, const u16 *q, const u16 *k, const u16 *v, const u16 *o,
                                           const float *den, int64_t t0, int64_t T, int tid) {
    const int64_t bytes = (T - t0) * D1 * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + t0 * D1, bytes), rk = make_rsrc(k + t0 * D1, bytes),
                                 rv = make_rsrc(v + t0 * D1, bytes), ro = make_rsrc(o + t0 * D1, bytes);
#pragma unroll
    for (int s = 0; s < NCH1; ++s) {
        const int cid = tid + s * kT1, off = ((cid / (D1 / 8)) * D1 + (cid % (D1 / 8)) * 8) * 2;
        r.q[s] = bload(rq, off);
        r.k[s] = bload(rk, off);
        r.v[s] = bload(rv, off);
        r.o[s] = bload(ro, off);
        if constexpr (DS) {
            const int64_t t = t0 + cid / (D1 / 8);
            r.den[s] = t < T ? den[t] : 1.0f;   // rows past the end are zeros
        }
    }
}

template <bool DS = false>
__device__ __forceinline__ void store_tile1(const Staged1 &r, u16 *smem, int tid) {
#pragma unroll
    for (int s = 0; s < NCH1; ++s) {
        const int cid = tid + s * kT1, off = nat_off<D1>(cid / (D1 / 8), cid % (D1 / 8));
        lds_write(smem + oQ1, off, r.q[s]);
        lds_write(smem + oK1, off, r.k[s]);
        lds_write(smem + oV1, off, r.v[s]);
        u32x4 o = r.o[s];
        if constexpr (DS) {
            const float rd = 1.0f / r.den[s];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_bf16(__builtin_bit_cast(float, o[j] << 16) * rd,
                                 __builtin_bit_cast(float, o[j] & 0xffff0000u) * rd);
        }
        lds_write(smem + oO1, off, o);
    }
}

// One output unit of a wave: columns 64ch..64ch+63 of the output rows in block `orow`.
//   DV: rows s of dV; scores Q[t] . K[s] for t >= s; value dO; inter R^T K^T (R^T rows read plain)
//   DK: rows s of dK; scores dO[t] . V[s] for t >= s; value Q; inter R V^T
//   DQ: rows t of dQ; scores V[s] . dO[t] for s <= t; value K; inter S dO^T
template <Unit U, bool DEC = false, bool NK = false>
__device__ __forceinline__ void out_unit(f32x16 (&oacc)[2], const u16 *smem, int orow, int ch, int lane,
                                         const LaneOff &L, const DecayW &dw) {
    const u16 *sB = smem + (U == Unit::DV ? oK1 : U == Unit::DK ? oV1 : oO1);   // output-row role
    const u16 *sA = smem + (U == Unit::DV ? oQ1 : U == Unit::DK ? oO1 : oV1);   // source-row role
    const u16 *sC = smem + (U == Unit::DV ? oO1 : U == Unit::DK ? oQ1 : oK1);   // value role
    const u16 *sSt = smem + (U == Unit::DQ ? oST1 : oRT1);
    constexpr bool ADD = NK && U == Unit::DK;
    unit_products<U == Unit::DQ, U == Unit::DV, false, DEC, ADD>(
        oacc, sB, sA, sC, sSt, orow, ch, lane, L, nullptr, nullptr, dw,
        ADD ? reinterpret_cast<const float *>(smem + oDD1) : nullptr);
}

// NK: the DK unit's accumulators (rows s of block orow, columns 64ch..64ch+63) plus y, times phi'(k_s)
// (elu + 1: min(phi(k), 1) from the phi(k) tile; the identity: 1).  Entries 4q..4q+3 of acc[n] are
// columns 32n + 8q + 4h .. + 3 of the unit.
__device__ __forceinline__ void nk_finish(f32x16 (&oacc)[2], const u16 *smem, int orow, int ch, int lane, bool elu) {
    const int h = lane >> 5, col = lane & 31;
    const float *sY = reinterpret_cast<const float *>(smem + oY1);
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c0 = 64 * ch + 32 * n + 8 * q + 4 * h;
            const float4 y = *reinterpret_cast<const float4 *>(sY + c0);
            float g[4] = {oacc[n][4 * q] + y.x, oacc[n][4 * q + 1] + y.y, oacc[n][4 * q + 2] + y.z,
                          oacc[n][4 * q + 3] + y.w};
            if (elu) {
                const u32x2 kk = *reinterpret_cast<const u32x2 *>(smem + oK1 + nat_off<D1>(orow * 32 + col, c0 >> 3) +
                                                                  (c0 & 7));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const unsigned int w = kk[j >> 1];
                    const float pk = __builtin_bit_cast(float, (j & 1) ? (w & 0xffff0000u) : (w << 16));
                    g[j] *= fminf(pk, 1.0f);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) oacc[n][4 * q + j] = g[j];
        }
}

__device__ __forceinline__ float chain_l2(const Bwd1Args &p, int chain) {
    return p.decay != nullptr ? log2f(p.decay[chain % p.H]) : 0.0f;
}

// The tiles of one (chain, segment), walked from the last to the first.
struct Walk1 {
    int64_t T, tile_hi, base;
    int ntiles;
    __device__ int64_t t0(int it) const { return (tile_hi - 1 - it) * TB1; }
};

__device__ __forceinline__ Walk1 walk_of(const Bwd1Args &p, int chain, int seg) {
    Walk1 w;
    w.T = p.T;
    const int64_t NT = (p.T + TB1 - 1) / TB1, tile_lo = (int64_t)seg * p.seg_tiles;
    w.tile_hi = min(tile_lo + p.seg_tiles, NT);
    w.ntiles = (int)(w.tile_hi - tile_lo);
    w.base = (int64_t)chain * p.T * D1;
    return w;
}

// Producer wave: state blocks with rows kb in {2ch, 2ch + 1} of R (SK = false) or S (SK = true).
// R_b = R_{b+1} + Q_b^T dO_b is formed at the top of tile b but published as R^T only after barrier
// Y (dV and dK of tile b use R_{b+1}); S_{b-1} = S_b - K_b^T V_b is published before Y for dQ.
// Without dQ (ONE = false) the S producers hold no state and only stage their part of each tile.
template <bool SK, bool ONE, bool DEC, bool NK>
__device__ __forceinline__ void producer(const Bwd1Args &p, u16 *smem, int chain, int seg, int ch, int lane) {
    constexpr bool HOLD = ONE || !SK;   // this wave holds a state
    constexpr bool YR = NK && !SK;              // NK: this wave carries its 64 entries of y
    constexpr bool DDS = NK && SK;              // NK: wave 6 stages each tile's dden
    const Walk1 w = walk_of(p, chain, seg);
    const int kb0 = 2 * ch, tid = threadIdx.x;
    const int h = lane >> 5, col = lane & 31;
    const unsigned int sign = SK ? 0x80008000u : 0u;   // S is updated with -K
    const LaneOff L = lane_offsets(lane, ch);
    const u16 *gq = static_cast<const u16 *>(p.q) + w.base, *gk = static_cast<const u16 *>(p.k) + w.base;
    const u16 *gv = static_cast<const u16 *>(p.v) + w.base, *go = static_cast<const u16 *>(p.dout) + w.base;
    const float *gden = NK ? p.den + (int64_t)chain * p.T : nullptr;
    // R at the segment's end (0 for the last segment), S after the segment's last position
    const float *g = nullptr;
    if (SK && ONE)
        g = seg < p.nseg - 1 ? p.s_states + ((int64_t)chain * p.s_nsub + (seg + 1) * p.s_sub) * D1 * D1
                             : p.s_final + (int64_t)chain * D1 * D1;
    else if (!SK && seg < p.nseg - 1)
        g = p.r_states + ((int64_t)chain * p.r_nsub + state_index(seg, p.r_sub, p.r_nsub, true)) * D1 * D1;

    f32x16 sacc[HOLD ? 8 : 1];
    if constexpr (HOLD) {
        if (!SK && g != nullptr && p.r_compose) {
            // R at the segment's end from the deltas of the later pieces: run = lam^L run + dR[piece],
            // from the chain's last piece down to the one after this segment (the segment prefix's
            // recurrence, in the same order and fused multiply-adds)
            const float f = DEC ? exp2f((float)p.r_piece_len * chain_l2(p, chain)) : 1.0f;
            const int first = state_index(seg, p.r_sub, p.r_nsub, true) + 1;
            const float *base = p.r_states + (int64_t)chain * p.r_nsub * D1 * D1;
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[s][r] = 0.0f;
            for (int pc = p.r_nsub - 1; pc >= first; --pc) {
                const float *gd = base + (int64_t)pc * D1 * D1;
                // two blocks' 32 loads in flight at a time (left to itself the compiler waits for each)
#pragma unroll
                for (int s0 = 0; s0 < 8; s0 += 2) {
                    float t[2][16];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int kb = kb0 + (s0 + u) / 4, nb = (s0 + u) % 4;
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            t[u][r] = gd[(int64_t)(kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * D1 + nb * 32 + col];
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[s0 + u][r] = fmaf(f, sacc[s0 + u][r], t[u][r]);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int kb = kb0 + s / 4, nb = s % 4;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    sacc[s][r] = g != nullptr ? g[(int64_t)d * D1 + nb * 32 + col] : 0.0f;
                }
            }
        }
    }
    // a decay: lam^64 per tile on R, and lam^j on the Q^T operand's position j = 16x + 8h + e
    float wq[DEC ? TB1 / 16 : 1][8], lam64 = 1.0f;
    if constexpr (DEC) {
        const float l2 = chain_l2(p, chain);
        lam64 = exp2f(64.0f * l2);
#pragma unroll
        for (int x = 0; x < TB1 / 16; ++x)
#pragma unroll
            for (int e = 0; e < 8; ++e) wq[x][e] = exp2f(l2 * (float)(16 * x + 8 * h + e));
    }
    // the blocks as R^T or S^T (bf16, [d_v][d]) into LDS: accumulator entries 4g..4g+3 of a lane are
    // four consecutive d of one d_v row, one 8-byte write
    // NK: y of state rows d = 32(kb0 + i) + col (fp32, the same in both halves of the wave), and the
    // next tile's dden (one position per lane) for wave 6
    float ytot[YR ? 2 : 1] = {}, ddn = 0.0f;
    const float *gdd = DDS ? p.dden + (int64_t)chain * p.T : nullptr;
    auto load_dd = [&](int64_t t0) {
        if constexpr (DDS) ddn = ch == 0 && t0 + lane < w.T ? gdd[t0 + lane] : 0.0f;
    };
    auto store_dd = [&]() {
        if constexpr (DDS)
            if (ch == 0) reinterpret_cast<float *>(smem + oDD1)[lane] = ddn;
    };
    auto write_y = [&]() {
        if constexpr (YR)
            if (h == 0) {
                float *sY = reinterpret_cast<float *>(smem + oY1);
                sY[kb0 * 32 + col] = ytot[0];
                sY[(kb0 + 1) * 32 + col] = ytot[1];
            }
    };
    auto write_state = [&]() {
        if constexpr (!HOLD) return;
        u16 *dst = smem + (SK ? oST1 : oRT1);
#pragma unroll
        for (int s = 0; s < (HOLD ? 8 : 0); ++s)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 v = {pack_bf16(sacc[s][4 * q], sacc[s][4 * q + 1]),
                                 pack_bf16(sacc[s][4 * q + 2], sacc[s][4 * q + 3])};
                lds_write8(dst, (s % 4) * 32 * D1 + L.pw[s / 4][q], v);
            }
    };

    Staged1 st;
    load_tile1<NK>(st, gq, gk, gv, go, gden, w.t0(0), w.T, tid);
    load_dd(w.t0(0));
    store_tile1<NK>(st, smem, tid);
    store_dd();
    if (!SK) write_state();
    write_y();
    lds_barrier();   // X: the first tile and R^T

    for (int it = 0; it < w.ntiles; ++it) {
        const bool more = it + 1 < w.ntiles;
        // R += Q^T dO, or S -= K^T V; each operand fragment is read once per 16 positions and shared
        // by the blocks that use it
        if constexpr (HOLD) {
            const u16 *sA = smem + (SK ? oK1 : oQ1), *sC = smem + (SK ? oV1 : oO1);
            if constexpr (DEC) {
#pragma unroll
                for (int s = 0; s < 8; ++s)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[s][r] *= lam64;
            }
            float ypart[YR ? 2 : 1] = {};
#pragma unroll
            for (int x = 0; x < TB1 / 16; ++x) {
                bf16x8 fa[2], fc[4];
                float dd[YR ? 8 : 1];
                if constexpr (YR) {
                    // dden at the positions 16x + 8h + e of the fragments' elements e
                    const float *sDd = reinterpret_cast<const float *>(smem + oDD1) + 16 * x + 8 * h;
                    const float4 a0 = *reinterpret_cast<const float4 *>(sDd),
                                 a1 = *reinterpret_cast<const float4 *>(sDd + 4);
                    dd[0] = a0.x, dd[1] = a0.y, dd[2] = a0.z, dd[3] = a0.w;
                    dd[4] = a1.x, dd[5] = a1.y, dd[6] = a1.z, dd[7] = a1.w;
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {   // state row blocks kb0 + i are column blocks 2ch + i of the tile
                    fa[i] = flip8(rd_tr(sA, 16 * x, L.trc[0][i]), sign);
                    if constexpr (YR) {
                        const u32x4 u = __builtin_bit_cast(u32x4, fa[i]);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            ypart[i] += dd[2 * j] * __builtin_bit_cast(float, u[j] << 16) +
                                        dd[2 * j + 1] * __builtin_bit_cast(float, u[j] & 0xffff0000u);
                    }
                    if constexpr (DEC) {
                        u32x4 u = __builtin_bit_cast(u32x4, fa[i]);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            u[j] = pack_bf16(__builtin_bit_cast(float, u[j] << 16) * wq[x][2 * j],
                                             __builtin_bit_cast(float, u[j] & 0xffff0000u) * wq[x][2 * j + 1]);
                        fa[i] = __builtin_bit_cast(bf16x8, u);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) fc[i] = rd_tr(sC, 16 * x, L.trn[i]);
#pragma unroll
                for (int s = 0; s < 8; ++s) sacc[s] = mfma(fa[s / 4], fc[s % 4], sacc[s]);
            }
            if constexpr (YR) {
                // the two halves of the wave hold positions 8h.. of every 16: add the partner's
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const unsigned int yu = __builtin_bit_cast(unsigned int, ypart[i]);
                    const auto r = __builtin_amdgcn_permlane32_swap(yu, yu, false, false);
                    ytot[i] += __builtin_bit_cast(float, (unsigned int)r[0]) +
                               __builtin_bit_cast(float, (unsigned int)r[1]);
                }
            }
        }
        if (SK) write_state();
        // this wave's part of the next tile: in flight while the consumers form this tile's gradients
        if (more) {
            load_tile1<NK>(st, gq, gk, gv, go, gden, w.t0(it + 1), w.T, tid);
            load_dd(w.t0(it + 1));
        }
        lds_barrier();   // Y
        if (!SK) write_state();
        write_y();
        lds_barrier();   // Z
        if (more) {
            store_tile1<NK>(st, smem, tid);
            store_dd();
        }
        lds_barrier();   // X
    }
}

// Consumer wave c = 2rb + ch.  Each unit is staged in the wave's own 8 KiB of LDS and stored as whole
// 128-byte row pieces, so that at most one unit's accumulators are held at a time.
template <bool ONE, bool DEC, bool NK>
__device__ __forceinline__ void consumer(const Bwd1Args &p, u16 *smem, int chain, int seg, int c, int lane) {
    const Walk1 w = walk_of(p, chain, seg);
    const int rb = c >> 1, ch = c & 1, tid = threadIdx.x;
    const LaneOff L = lane_offsets(lane, ch);
    const u16 *gq = static_cast<const u16 *>(p.q) + w.base, *gk = static_cast<const u16 *>(p.k) + w.base;
    const u16 *gv = static_cast<const u16 *>(p.v) + w.base, *go = static_cast<const u16 *>(p.dout) + w.base;
    const float *gden = NK ? p.den + (int64_t)chain * p.T : nullptr;
    u16 *gdq = static_cast<u16 *>(p.dq) + w.base, *gdk = static_cast<u16 *>(p.dk) + w.base,
        *gdv = static_cast<u16 *>(p.dv) + w.base;
    u16 *ob = smem + oOS1 + c * kOS1;
    DecayW dwt = {};   // read only with a decay
    if constexpr (DEC) dwt = decay_weights<false>(chain_l2(p, chain), rb, lane);
    // [32 rows][64 columns] with 16-byte chunks XOR-swizzled by row pair; a lane's accumulator entries
    // 4g..4g+3 are four consecutive columns of its row, one 8-byte write
    auto stage = [&](const f32x16 (&acc)[2], u16 *dst) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 v = {pack_bf16(acc[n][4 * q], acc[n][4 * q + 1]),
                                 pack_bf16(acc[n][4 * q + 2], acc[n][4 * q + 3])};
                lds_write8(dst, L.po[n][q], v);
            }
    };
    auto store = [&](const u16 *src, u16 *g, int64_t t0) {
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(g + t0 * D1, (w.T - t0) * D1 * 2);
        u32x4 v[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int qd = lane + 64 * s2, row = qd / 8, chk = qd % 8;
            v[s2] = *reinterpret_cast<const u32x4 *>(src + row * 64 + ((chk ^ ((row >> 1) & 7)) << 3));
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int qd = lane + 64 * s2, row = qd / 8, chk = qd % 8;
            bstore16(ry, ((rb * 32 + row) * D1 + ch * 64 + chk * 8) * 2, v[s2]);
        }
    };

    Staged1 st;
    load_tile1<NK>(st, gq, gk, gv, go, gden, w.t0(0), w.T, tid);
    store_tile1<NK>(st, smem, tid);
    lds_barrier();   // X: the first tile and R^T
    for (int it = 0; it < w.ntiles; ++it) {
        const int64_t t0 = w.t0(it);
        const bool more = it + 1 < w.ntiles;
        // this wave's part of the next tile
        if (more) load_tile1<NK>(st, gq, gk, gv, go, gden, w.t0(it + 1), w.T, tid);
        {
            f32x16 oacc[2];
            out_unit<Unit::DV, DEC>(oacc, smem, rb, ch, lane, L, dwt);
            stage(oacc, ob);
            out_unit<Unit::DK, DEC, NK>(oacc, smem, rb, ch, lane, L, dwt);
            if constexpr (NK) nk_finish(oacc, smem, rb, ch, lane, p.nk_elu != 0);
            stage(oacc, ob + 2048);
            store(ob, gdv, t0);
            store(ob + 2048, gdk, t0);
        }
        lds_barrier();   // Y: S^T of the state before this tile is complete
        if constexpr (ONE) {
            f32x16 oacc[2];
            out_unit<Unit::DQ>(oacc, smem, rb, ch, lane, L, dwt);
            stage(oacc, ob);
        }
        lds_barrier();   // Z
        if (more) store_tile1<NK>(st, smem, tid);
        if constexpr (ONE) store(ob, gdq, t0);
        lds_barrier();   // X
    }
}

template <bool ONE, bool DEC, bool NK = false>
__global__ __launch_bounds__(kT1, 1) void bwd1_bf16_kernel(Bwd1Args p) {
    static_assert(!NK || (!ONE && !DEC), "the normalized dk terms ride on the dK/dV walk without decay");
    __shared__ __attribute__((aligned(16))) u16 smem[kLds1];
    // the wave index as a scalar: every branch on a wave's role is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int seg = blockIdx.x % p.nseg;
    const int chain = blockIdx.x / p.nseg;
    const int64_t NT = (p.T + TB1 - 1) / TB1;
    if ((int64_t)seg * p.seg_tiles >= NT) return;
    if (wave < 4)
        consumer<ONE, DEC, NK>(p, smem, chain, seg, wave, lane);
    else if (wave < 6)
        producer<false, ONE, DEC, NK>(p, smem, chain, seg, wave & 1, lane);
    else
        producer<true, ONE, DEC, NK>(p, smem, chain, seg, wave & 1, lane);
}

}  // namespace

hipError_t launch_bwd1_bf16(const Bwd1Args &a, hipStream_t s) {
    const unsigned items = (unsigned)((int64_t)a.chains * a.nseg);
    if (a.dq != nullptr && a.decay != nullptr) return hipErrorInvalidValue;   // no one-pass walk with a decay
    if (a.decay != nullptr && a.H <= 0) return hipErrorInvalidValue;
    if (a.r_compose && (a.r_states == nullptr || a.r_piece_len <= 0 || a.r_sub <= 0 || a.r_nsub <= 0))
        return hipErrorInvalidValue;
    if (a.dden != nullptr) {
        // y starts from zero at the chain's end: unsplit chains only
        if (a.dq != nullptr || a.decay != nullptr || a.nseg != 1 || a.r_states != nullptr || a.den == nullptr)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd1_bf16_kernel<false, false, true>), dim3(items), dim3(kT1), 0, s, a);
        return hipGetLastError();
    }
    if (a.dq != nullptr)
        hipLaunchKernelGGL((bwd1_bf16_kernel<true, false>), dim3(items), dim3(kT1), 0, s, a);
    else if (a.decay != nullptr)
        hipLaunchKernelGGL((bwd1_bf16_kernel<false, true>), dim3(items), dim3(kT1), 0, s, a);
    else
        hipLaunchKernelGGL((bwd1_bf16_kernel<false, false>), dim3(items), dim3(kT1), 0, s, a);
    return hipGetLastError();
}

}  // namespace la2
