// la2_dkdv_bf16.hip -- fused reverse pass of the Lightning Attention-2 backward on gfx950 MFMA:
// dK and dV of one (chain, segment) in a single walk over its tiles, last to first.
//
// Both gradients are reverse scans that share one state (page "Lightning Attention",
// lizeman.github.io llm-arch-kb, section 2, Steps 1-4, run backwards).  The optional per-head decay
// lam is not defined on the pages; it enters through the token recurrence S_t = lam S_{t-1} +
// k_t v_t^T, whose chain-rule backward is:
//   R_t  = lam R_{t+1} + q_t do_t^T                 (d x d_v, fp32 in MFMA accumulators)
//   dk_t = R_t v_t,   dv_t = R_t^T k_t
// Per tile of TB positions, with local rows i (outputs) and j (sources), j >= i inside the tile:
//   dV_b^T = R^T K_b^T diag(w) + dO_b^T P_v^T,   P_v^T = mask(Q_b K_b^T)   [j][i] = q_j . k_i
//   dK_b^T = R   V_b^T diag(w) + Q_b^T  P_k^T,   P_k^T = mask(dO_b V_b^T)  [j][i] = do_j . v_i
//   R      = lam^TB R + (diag(w_upd) Q_b)^T dO_b
// with mask lam^(j-i) for j >= i, w = lam^(TB-i), w_upd = lam^j.  Reading q, k, v and dO once for
// both gradients moves 6 tensors per token instead of the 8 of two separate reverse scans, and the
// state update is done once.  R^T is kept in LDS as bf16 once: the dV waves read it with plain
// fragment reads, the dK waves read R through transpose reads.
//
// Workgroup of 8 waves, TB = 64 (two 32-row blocks): waves 0-3 produce dV, waves 4-7 dK; each
// wave owns one row block and half the columns.  Wave w and w + 4 share a SIMD and get opposite
// row blocks, so every SIMD has one long and one short causal block.  d = d_v in {64, 128}.
#include <type_traits>

#include "la2_bf16_common.h"

namespace la2 {
namespace {

using namespace dev;

template <int D, bool DECAY>
struct FCfg {
    static constexpr int TB = kDkdvTile;
    static constexpr int NTB = TB / 32;          // row blocks of a tile
    static constexpr int NDB = D / 32;           // 32-column blocks of an output
    static constexpr int ODB = NDB / 2;          // column blocks per wave
    static constexpr int KS = D / 16;            // contraction steps over d
    static constexpr int NSB = NDB * NDB;        // 32x32 blocks of R
    static constexpr int SPW = NSB >= kWaves ? NSB / kWaves : 1;
    static constexpr int TE = TB * D;            // elements of one tile
    static constexpr int NCH = TE / 8 / kThreads;   // 16-byte chunks per thread and tile
    // LDS (bf16 elements): the four tiles, R^T, the weighted Q copy (decay), per-wave output staging
    static constexpr int oQ = 0, oK = TE, oV = 2 * TE, oO = 3 * TE;
    static constexpr int oST = 4 * TE;
    static constexpr int oQW = oST + D * D;
    static constexpr int OSW = ODB * 32;
    static constexpr int oOS = oQW + (DECAY ? TE : 0);
    static constexpr int kLds = oOS + kWaves * 32 * OSW;
    static_assert(NTB == 2 && NDB >= 2, "two row blocks, two column halves");
    static_assert(NCH >= 1 && NCH * 8 * kThreads == TE, "whole chunks per thread");
    static_assert(SPW * kWaves == NSB || (SPW == 1 && NSB <= kWaves), "state blocks");
    static_assert(kLds * 2 <= 160 * 1024, "LDS");
};

template <int D>
struct FStaged {
    static constexpr int NCH = FCfg<D, false>::NCH;
    u32x4 q[NCH], k[NCH], v[NCH], o[NCH];
};

// Global loads of the four tiles starting at t0 into registers; rows at or past T read as zero.
// PART: 0 all four, 1 Q and dO only, 2 K and V only.
template <int D, int PART = 0>
__device__ __forceinline__ void fstage_load(FStaged<D> &r, const u16 *q, const u16 *k, const u16 *v, const u16 *o,
                                            int64_t t0, int64_t T, int tid) {
    const int64_t bytes = (T - t0) * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + t0 * D, bytes), rk = make_rsrc(k + t0 * D, bytes),
                                 rv = make_rsrc(v + t0 * D, bytes), ro = make_rsrc(o + t0 * D, bytes);
#pragma unroll
    for (int s = 0; s < FStaged<D>::NCH; ++s) {
        const int cid = tid + s * kThreads, off = ((cid / (D / 8)) * D + (cid % (D / 8)) * 8) * 2;
        if constexpr (PART != 2) r.q[s] = bload(rq, off);
        if constexpr (PART != 1) r.k[s] = bload(rk, off);
        if constexpr (PART != 1) r.v[s] = bload(rv, off);
        if constexpr (PART != 2) r.o[s] = bload(ro, off);
    }
}

template <int D, bool DECAY>
__device__ __forceinline__ void fstage_store(const FStaged<D> &r, u16 *smem, int tid, float l2) {
    using C = FCfg<D, DECAY>;
#pragma unroll
    for (int s = 0; s < C::NCH; ++s) {
        const int cid = tid + s * kThreads, row = cid / (D / 8), off = nat_off<D>(row, cid % (D / 8));
        lds_write(smem + C::oQ, off, r.q[s]);
        lds_write(smem + C::oK, off, r.k[s]);
        lds_write(smem + C::oV, off, r.v[s]);
        lds_write(smem + C::oO, off, r.o[s]);
        if constexpr (DECAY) {
            // the state update's copy of Q: row j scaled by w_upd(j) = lam^j, rounded once to bf16
            const float w = __builtin_amdgcn_exp2f((float)row * l2);
            u32x4 x = r.q[s];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                x[m] = f32_to_bf16(__uint_as_float(x[m] << 16) * w) |
                       (f32_to_bf16(__uint_as_float(x[m] & 0xffff0000u) * w) << 16);
            lds_write(smem + C::oQW, off, x);
        }
    }
}

template <int D, bool DECAY>
__global__ __launch_bounds__(kThreads, 1) void dkdv_bf16_kernel(DkdvArgs p) {
    using C = FCfg<D, DECAY>;
    constexpr int TB = C::TB;
    __shared__ __attribute__((aligned(16))) u16 smem[C::kLds];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;

    const int seg = blockIdx.x % p.nseg;
    const int chain = blockIdx.x / p.nseg;
    const int64_t T = p.T;
    const int64_t NT = (T + TB - 1) / TB;
    const int64_t tile_lo = (int64_t)seg * p.seg_tiles;
    const int64_t tile_hi = min(tile_lo + p.seg_tiles, NT);
    if (tile_lo >= tile_hi) return;
    const int ntiles = (int)(tile_hi - tile_lo);

    const int64_t base = (int64_t)chain * T * D;
    const u16 *gq = static_cast<const u16 *>(p.q) + base, *gk = static_cast<const u16 *>(p.k) + base;
    const u16 *gv = static_cast<const u16 *>(p.v) + base, *go = static_cast<const u16 *>(p.dout) + base;
    u16 *gdk = static_cast<u16 *>(p.dk) + base, *gdv = static_cast<u16 *>(p.dv) + base;
    const float *gs =
        p.states ? p.states + ((int64_t)chain * p.nsub + state_index(seg, p.sub, p.nsub, true)) * D * D : nullptr;

    const float l2 = DECAY ? log2f(p.decay[chain % p.H]) : 0.0f;
    auto pw = [&](int n) -> float { return DECAY ? __builtin_amdgcn_exp2f((float)n * l2) : 1.0f; };

    // roles: waves 0-3 dV, 4-7 dK; row block tb, column blocks db0 .. db0 + ODB - 1
    const bool is_dk = wave >= 4;
    const int w4 = wave & 3;
    const int tb = is_dk ? 1 - (w4 & 1) : (w4 & 1);
    const int db0 = (w4 >> 1) * C::ODB;
    const bool s_active = wave * C::SPW < C::NSB;

    // R blocks (d rows kb, d_v columns nb), fp32; segment start state when the chain is split
    f32x16 sacc[C::SPW];
    const bool init_state = gs != nullptr && (seg < p.nseg - 1 || p.has_init);
    // a carried-in R (gradient of a carried-out forward state) is attached at the chain's last
    // position: on the chain's last tile, the first processed here, rows are weighted lam^(leff-1-i)
    // and it is carried on with lam^(leff-1), leff the tile's real length
    const bool end_init = p.has_init && seg == p.nseg - 1;
    const int leff_end = (int)min((int64_t)TB, T - (NT - 1) * TB);
#pragma unroll
    for (int s = 0; s < C::SPW; ++s) {
        const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            sacc[s][r] = (init_state && s_active) ? gs[(int64_t)d * D + nb * 32 + col] : 0.0f;
        }
    }

    // R^T (bf16, [d_v][d]) into LDS for the next tile's inter products
    auto write_state_lds = [&]() {
        if (!s_active) return;
#pragma unroll
        for (int s = 0; s < C::SPW; ++s) {
            const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
            // the halves of chunks j = 2jp and 2jp + 1 (d = kb*32 + 8j + 4h + 0..3) are paired across h,
            // so each lane writes one whole 16-byte chunk (no bank conflicts)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                u32x2 a, b;
                a[0] = pack_bf16(sacc[s][8 * jp + 0], sacc[s][8 * jp + 1]);
                a[1] = pack_bf16(sacc[s][8 * jp + 2], sacc[s][8 * jp + 3]);
                b[0] = pack_bf16(sacc[s][8 * jp + 4], sacc[s][8 * jp + 5]);
                b[1] = pack_bf16(sacc[s][8 * jp + 6], sacc[s][8 * jp + 7]);
                lds_write(smem + C::oST, nat_off<D>(nb * 32 + col, kb * 4 + 2 * jp + h), join_halves(a, b));
            }
        }
    };

    auto tile_of = [&](int it) -> int64_t { return tile_hi - 1 - it; };

    FStaged<D> st;
    fstage_load<D>(st, gq, gk, gv, go, tile_of(0) * TB, T, tid);
    fstage_store<D, DECAY>(st, smem, tid, l2);
    if (init_state) write_state_lds();
    lds_barrier();

    const u16 *sQ = smem + C::oQ, *sK = smem + C::oK, *sV = smem + C::oV, *sO = smem + C::oO;
    const u16 *sST = smem + C::oST;
    bool state_nonzero = init_state;

    // One wave's output block for the tile at t0.  DK selects the gradient: the rows of the
    // tile's "query" role (B operand of the scores, rows tb) are K for dV and V for dK, the
    // "key" role (rows u) Q for dV and dO for dK, and the "value" role dO for dV and Q for dK.
    auto out_block = [&](auto dk_tag, int64_t t0, bool first_end) __attribute__((always_inline)) {
        constexpr bool DK = decltype(dk_tag)::value;
        const u16 *sB = DK ? sV : sK;
        const u16 *sA = DK ? sO : sQ;
        const u16 *sC = DK ? sQ : sO;
        u16 *gy = DK ? gdk : gdv;
        const int brow = tb * 32 + col;
        auto rdB = [&](int ks) { return lds_read(sB, nat_off<D>(brow, 2 * ks + h)); };
        // inter-product A operand: R^T rows (dV, plain reads) or R rows (dK, transpose reads of R^T)
        auto rdS = [&](int n, int ks) {
            if constexpr (DK)
                return frag_tr<D, false>(sST, 16 * ks, (db0 + n) * 32, lane);
            else
                return lds_read(sST, nat_off<D>((db0 + n) * 32 + col, 2 * ks + h));
        };

        f32x16 oacc[C::ODB];
#pragma unroll
        for (int n = 0; n < C::ODB; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0f;

        if (state_nonzero) {
            bf16x8 ba = rdB(0), sa[C::ODB];
#pragma unroll
            for (int n = 0; n < C::ODB; ++n) sa[n] = rdS(n, 0);
#pragma unroll 2
            for (int ks = 0; ks < C::KS; ++ks) {
                const int kn = ks + 1 < C::KS ? ks + 1 : ks;
                const bf16x8 bn = rdB(kn);
                bf16x8 sn[C::ODB];
#pragma unroll
                for (int n = 0; n < C::ODB; ++n) sn[n] = rdS(n, kn);
#pragma unroll
                for (int n = 0; n < C::ODB; ++n) oacc[n] = mfma(sa[n], ba, oacc[n]);
                ba = bn;
#pragma unroll
                for (int n = 0; n < C::ODB; ++n) sa[n] = sn[n];
            }
            if constexpr (DECAY) {
                const int ew = first_end ? leff_end - 1 - brow : TB - brow;
                const float w = ew >= 0 ? pw(ew) : 0.0f;
#pragma unroll
                for (int n = 0; n < C::ODB; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[n][r] *= w;
            }
        }

        // intra-tile: source blocks u >= tb (reverse causality)
        for (int u = tb; u < C::NTB; ++u) {
            asm volatile("" ::: "memory");
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            bf16x8 aa = lds_read(sA, nat_off<D>(u * 32 + col, h)), ba = rdB(0);
#pragma unroll
            for (int ks = 0; ks < C::KS; ks += 2) {
                const bf16x8 ab = lds_read(sA, nat_off<D>(u * 32 + col, 2 * (ks + 1) + h)), bb = rdB(ks + 1);
                acc = mfma(aa, ba, acc);
                if (ks + 2 < C::KS) {
                    aa = lds_read(sA, nat_off<D>(u * 32 + col, 2 * (ks + 2) + h));
                    ba = rdB(ks + 2);
                }
                acc = mfma(ab, bb, acc);
            }
            // mask lam^(j-i) for j >= i; only the diagonal block has masked entries.  The weights are
            // recomputed per block (hiding log2 lam from loop-invariant hoisting): kept across the
            // tile loop they would be spilled, and every reload waits on the next tile's loads.
            // j - i of accumulator r is base + 8 (r / 4) + r % 4 (small integers, exact in fp32)
            float base = (float)(u * 32 + 4 * h - brow);
            asm volatile("" : "+v"(base));
            bf16x8 pf[2];
            if (DECAY && u != tb) {
                // off the diagonal every distance is >= 1: lam^dist = lam^(base + 8m) * lam^e, one exp
                // per group of 4 accumulators, both exponents >= 0 (lam^e rebuilt per block from a
                // hidden copy of log2 lam rather than held across the tile loop)
                float l2b = l2;
                asm volatile("" : "+v"(l2b));
                const float lam_e[4] = {1.0f, __builtin_amdgcn_exp2f(l2b), __builtin_amdgcn_exp2f(2.0f * l2b),
                                        __builtin_amdgcn_exp2f(3.0f * l2b)};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float pm = __builtin_amdgcn_exp2f((base + (float)(8 * m)) * l2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pf[m >> 1][4 * (m & 1) + e] = (__bf16)(acc[4 * m + e] * (pm * lam_e[e]));
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float diff = base + (float)(8 * (r >> 2) + (r & 3));
                    const float w = DECAY ? __builtin_amdgcn_exp2f(diff * l2) : 1.0f;
                    const float v = diff >= 0.0f ? (DECAY ? acc[r] * w : acc[r]) : 0.0f;
                    pf[r >> 3][r & 7] = (__bf16)v;
                }
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int n = 0; n < C::ODB; ++n)
                    oacc[n] = mfma(frag_tr<D, true>(sC, u * 32 + 16 * x, (db0 + n) * 32, lane), pf[x], oacc[n]);
        }

        // store through this wave's LDS block: whole 16-byte row pieces per lane
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(gy + t0 * D, (T - t0) * D * 2);
        constexpr int NC = C::OSW / 8;
        u16 *ob = smem + C::oOS + wave * 32 * C::OSW;
        // 16 lanes writing one chunk of 16 consecutive rows (or reading whole rows) hit 16 bank groups
        auto oswz = [&](int row) { return (row / (16 / NC)) & (NC - 1); };
#pragma unroll
        for (int n = 0; n < C::ODB; ++n)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                u32x2 a, b;
                a[0] = pack_bf16(oacc[n][8 * jp + 0], oacc[n][8 * jp + 1]);
                a[1] = pack_bf16(oacc[n][8 * jp + 2], oacc[n][8 * jp + 3]);
                b[0] = pack_bf16(oacc[n][8 * jp + 4], oacc[n][8 * jp + 5]);
                b[1] = pack_bf16(oacc[n][8 * jp + 6], oacc[n][8 * jp + 7]);
                const int ch = 4 * n + 2 * jp + h;
                lds_write(ob, col * C::OSW + ((ch ^ oswz(col)) << 3), join_halves(a, b));
            }
#pragma unroll
        for (int s2 = 0; s2 < 32 * NC / 64; ++s2) {
            const int qd = lane + 64 * s2, row = qd / NC, ch = qd % NC;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + row * C::OSW + ((ch ^ oswz(row)) << 3));
            bstore16(ry, ((tb * 32 + row) * D + db0 * 32 + ch * 8) * 2, v);
        }
    };

    for (int it = 0; it < ntiles; ++it) {
        const int64_t t0 = tile_of(it) * TB;
        const bool update = it + 1 < ntiles;

        const bool first_end = end_init && it == 0;
        // the next tile's loads go out first and have the whole tile to land (32 VGPRs of staging fit
        // beside the output block's registers: no spills, measured ~1% faster than issuing them after
        // it); with decay, only K and V go out here and Q and dO after the output blocks (~1% faster
        // on the decay workloads)
        if (update) fstage_load<D, DECAY ? 2 : 0>(st, gq, gk, gv, go, tile_of(it + 1) * TB, T, tid);
        if (is_dk)
            out_block(std::true_type{}, t0, first_end);
        else
            out_block(std::false_type{}, t0, first_end);


        if constexpr (DECAY) {
            if (update) fstage_load<D, 1>(st, gq, gk, gv, go, tile_of(it + 1) * TB, T, tid);
        }
        // R = lam^TB R + (w_upd Q)^T dO
        if (update) {
            if (s_active) {
                if constexpr (DECAY) {
                    const float f = first_end ? pw(leff_end - 1) : pw(TB);
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) sacc[s] *= f;
                }
                const u16 *sQU = DECAY ? smem + C::oQW : sQ;
                auto rdQT = [&](int s, int x) {
                    return frag_tr<D, false>(sQU, 16 * x, ((wave * C::SPW + s) / C::NDB) * 32, lane);
                };
                auto rdO = [&](int s, int x) {
                    return frag_tr<D, false>(sO, 16 * x, ((wave * C::SPW + s) % C::NDB) * 32, lane);
                };
                bf16x8 qa[C::SPW], oa[C::SPW];
#pragma unroll
                for (int s = 0; s < C::SPW; ++s) {
                    qa[s] = rdQT(s, 0);
                    oa[s] = rdO(s, 0);
                }
#pragma unroll 2
                for (int x = 0; x < TB / 16; ++x) {
                    bf16x8 qn[C::SPW], on[C::SPW];
                    const int xn = x + 1 < TB / 16 ? x + 1 : x;
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) {
                        qn[s] = rdQT(s, xn);
                        on[s] = rdO(s, xn);
                    }
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) sacc[s] = mfma(qa[s], oa[s], sacc[s]);
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) {
                        qa[s] = qn[s];
                        oa[s] = on[s];
                    }
                }
            }
            state_nonzero = true;
        }

        lds_barrier();   // every wave is done with this tile's LDS
        if (update) {
            write_state_lds();
            fstage_store<D, DECAY>(st, smem, tid, l2);
        }
        lds_barrier();
    }

    // Gradient of a carried-in forward state: lam R_0, R_0 = lam^TB R + (w_upd Q)^T dO over tile 0
    // (the update the loop leaves out; the tile is still in LDS, rows past T are zero).
    if (p.state_out != nullptr && seg == 0 && s_active) {
        if constexpr (DECAY) {
            const float f = end_init && ntiles == 1 ? pw(leff_end - 1) : pw(TB);
#pragma unroll
            for (int s = 0; s < C::SPW; ++s) sacc[s] *= f;
        }
        const u16 *sQU = DECAY ? smem + C::oQW : sQ;
#pragma unroll
        for (int s = 0; s < C::SPW; ++s) {
            const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
            for (int x = 0; x < TB / 16; ++x)
                sacc[s] = mfma(frag_tr<D, false>(sQU, 16 * x, kb * 32, lane), frag_tr<D, false>(sO, 16 * x, nb * 32, lane),
                               sacc[s]);
            const float scale = pw(1);
            float *so = p.state_out + (int64_t)chain * D * D;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                so[(int64_t)d * D + nb * 32 + col] = sacc[s][r] * scale;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const DkdvArgs &a, hipStream_t s) {
    const unsigned items = (unsigned)((int64_t)a.chains * a.nseg);
    if (a.decay)
        hipLaunchKernelGGL((dkdv_bf16_kernel<D, true>), dim3(items), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((dkdv_bf16_kernel<D, false>), dim3(items), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool dkdv_supported(int D, int DV) { return D == DV && (D == 64 || D == 128); }

hipError_t launch_dkdv_bf16(const DkdvArgs &a, int D, hipStream_t s) {
    if (!dkdv_supported(D, D)) return hipErrorInvalidValue;
    return D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace la2
