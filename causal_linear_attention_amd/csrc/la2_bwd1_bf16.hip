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
// Workgroup of four waves (one per SIMD), 64-position tiles (two 32-row blocks).  Wave w = 2rb + ch
// produces columns 64ch..64ch+63 of dV and dK for row block rb and of dQ for row block 1 - rb (the
// causal block counts of those units differ, so that every wave has about the same work), and
// updates eight of the 32 state blocks: waves 0 and 1 half of R each, waves 2 and 3 half of S.  LDS
// holds the four input tiles, R^T and S^T in bf16 (MFMA operands of the inter-tile products) and
// 8 KiB of output staging per wave: 160 KiB.  The next tile's inputs are loaded into registers once
// the state updates are done and written to LDS at the end of the tile.
#include "la2_bf16_common.h"

namespace la2 {
namespace {

using namespace dev;

constexpr int D1 = 128;              // d = d_v
constexpr int TB1 = 64;              // positions per tile
constexpr int kW1 = 4;               // waves
constexpr int kT1 = 64 * kW1;        // threads
constexpr int kTile1 = TB1 * D1;     // bf16 elements of one input tile
constexpr int KS1 = D1 / 16;         // contraction steps over d
constexpr int oQ1 = 0, oK1 = kTile1, oV1 = 2 * kTile1, oO1 = 3 * kTile1;   // q, k, v, dO tiles
constexpr int oRT1 = 4 * kTile1;                                           // R^T [d_v][d] bf16
constexpr int oST1 = oRT1 + D1 * D1;                                       // S^T [d_v][d] bf16
constexpr int oOS1 = oST1 + D1 * D1;                                       // per-wave output staging
constexpr int kOS1 = 2 * 32 * 64;                                          //   (two units of 32 x 64)
constexpr int kLds1 = oOS1 + kW1 * kOS1;
constexpr int NCH1 = kTile1 / 8 / kT1;   // 16-byte chunks per thread and tile (4)
static_assert(kLds1 * 2 <= 160 * 1024, "LDS");


enum class Unit { DV, DK, DQ };

struct Staged1 {
    u32x4 q[NCH1], k[NCH1], v[NCH1], o[NCH1];
};

__device__ __forceinline__ void load_tile1(Staged1 &r, const u16 *q, const u16 *k, const u16 *v, const u16 *o,
                                           int64_t t0, int64_t T, int tid) {
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
    }
}

__device__ __forceinline__ void store_tile1(const Staged1 &r, u16 *smem, int tid) {
#pragma unroll
    for (int s = 0; s < NCH1; ++s) {
        const int cid = tid + s * kT1, off = nat_off<D1>(cid / (D1 / 8), cid % (D1 / 8));
        lds_write(smem + oQ1, off, r.q[s]);
        lds_write(smem + oK1, off, r.k[s]);
        lds_write(smem + oV1, off, r.v[s]);
        lds_write(smem + oO1, off, r.o[s]);
    }
}

// bf16x8 with every element negated (sign bits flipped: exact).
__device__ __forceinline__ bf16x8 neg8(const bf16x8 &f) {
    u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int m = 0; m < 4; ++m) u[m] ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, u);
}

// Per-lane LDS offsets (bf16 elements), computed once so that every LDS access in the tile loop is a
// per-lane register plus a compile-time or per-block offset.  Tiles are [rows][128] with 16-byte
// chunks XOR-swizzled by row (nat_off); the swizzle depends only on row % 16, so within a lane it is
// the same for every row block, and the chunk index splits into bits the block offset cannot carry.
struct LaneOff {
    int pl[8];          // row col, chunk 2m + h (plain fragment reads and state writes; + 128 row0)
    int trn[4][2];      // transposed reads without permutation at k0 = 0 of column block nb (+ 128 k0),
                        // first and second 8-byte piece
    int trc[2][2][2];   // [PERM][n][piece] the same for this wave's column blocks 2ch + n
    int pw[2][2];       // row col, chunk 4(2ch + i) + 2jp + h: where this wave's state
                        // block rows kb = 2ch + i land in a transposed state
};

__device__ __forceinline__ int tr_off(int lane, int perm, int half, int nb) {
    const int g = lane >> 4, j = lane & 15, hh = g >> 1;
    const int cl = 2 * (g & 1) + ((j & 3) >> 1);   // chunk bits below the column block's
    const int rl = (perm ? 4 * hh : 8 * hh) + (j >> 2) + (half ? (perm ? 8 : 4) : 0);
    const int S = swz<D1>(rl);
    return rl * D1 + ((((4 * nb) ^ (S & 12)) | (cl ^ (S & 3))) << 3) + 4 * (j & 1);
}

__device__ __forceinline__ LaneOff lane_offsets(int lane, int ch) {
    LaneOff L;
    const int h = lane >> 5, col = lane & 31;
#pragma unroll
    for (int m = 0; m < 8; ++m) L.pl[m] = nat_off<D1>(col, 2 * m + h);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int half = 0; half < 2; ++half) L.trn[nb][half] = tr_off(lane, 0, half, nb);
#pragma unroll
    for (int perm = 0; perm < 2; ++perm)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int half = 0; half < 2; ++half) L.trc[perm][n][half] = tr_off(lane, perm, half, 2 * ch + n);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) L.pw[i][jp] = nat_off<D1>(col, 4 * (2 * ch + i) + 2 * jp + h);
    return L;
}

// Fragment (either MFMA side) of rows row0 + col, 8 consecutive columns 16m + 8h.. of a tile.
__device__ __forceinline__ bf16x8 rd_plain(const u16 *s, int row0, int m, const LaneOff &L) {
    return lds_read(s, row0 * D1 + L.pl[m]);
}

// A transposing fragment (frag_tr) at k0 (a multiple of 16) from the two piece offsets `off`.
__device__ __forceinline__ bf16x8 rd_tr(const u16 *s, int k0, const int (&off)[2]) {
    const u32x2 a = __builtin_bit_cast(u32x2, tr_read(s, k0 * D1 + off[0]));
    const u32x2 b = __builtin_bit_cast(u32x2, tr_read(s, k0 * D1 + off[1]));
    const u32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// One output unit of a wave: columns 64ch..64ch+63 (two 32-column blocks) of the output rows in
// block `orow`, as O^T accumulators (lane col holds output row orow*32 + col).
//   DV: rows s of dV; scores Q[t] . K[s] for t >= s; value dO; inter R^T K^T
//   DK: rows s of dK; scores dO[t] . V[s] for t >= s; value Q; inter R V^T
//   DQ: rows t of dQ; scores V[s] . dO[t] for s <= t; value K; inter S dO^T
template <Unit U>
__device__ __forceinline__ void out_unit(f32x16 (&oacc)[2], const u16 *smem, int orow, int ch, int lane,
                                         const LaneOff &L, bool inter) {
    const int h = lane >> 5, col = lane & 31;
    const u16 *sB = smem + (U == Unit::DV ? oK1 : U == Unit::DK ? oV1 : oO1);   // output-row role
    const u16 *sA = smem + (U == Unit::DV ? oQ1 : U == Unit::DK ? oO1 : oV1);   // source-row role
    const u16 *sC = smem + (U == Unit::DV ? oO1 : U == Unit::DK ? oQ1 : oK1);   // value role
    const u16 *sSt = smem + (U == Unit::DQ ? oST1 : oRT1);
    bf16x8 bf[KS1];
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) bf[ks] = rd_plain(sB, orow * 32, ks, L);
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0f;
    if (inter) {
        // fully unrolled: bf[] must be indexed by constants (a runtime index into a register array is
        // lowered to chains of selects)
#pragma unroll
        for (int ks = 0; ks < KS1; ++ks)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int cb = 2 * ch + n;
                // DV: R^T rows (d_v) from plain reads; DK, DQ: R or S rows (d) through transpose reads
                const bf16x8 a = U == Unit::DV ? rd_plain(sSt, cb * 32, ks, L) : rd_tr(sSt, 16 * ks, L.trc[0][n]);
                oacc[n] = mfma(a, bf[ks], oacc[n]);
            }
    }
    // intra-tile: source blocks u (u >= orow for DV, DK; u <= orow for DQ)
    const int ulo = U == Unit::DQ ? 0 : orow;
    const int uhi = U == Unit::DQ ? orow : TB1 / 32 - 1;
    for (int u = ulo; u <= uhi; ++u) {
        asm volatile("" ::: "memory");
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS1; ++ks) acc = mfma(rd_plain(sA, u * 32, ks, L), bf[ks], acc);
        // accumulator r holds source row u*32 + 8(r/4) + 4h + r%4 for output row orow*32 + col; only the
        // diagonal block (u == orow) has entries on the wrong side of the causal mask
        bf16x8 pf[2];
        if (u == orow) {
            const int base = 4 * h - col;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dist = base + 8 * (r >> 2) + (r & 3);   // source - output
                const bool keep = U == Unit::DQ ? dist <= 0 : dist >= 0;
                pf[r >> 3][r & 7] = (__bf16)(keep ? acc[r] : 0.0f);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)acc[r];
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int n = 0; n < 2; ++n) oacc[n] = mfma(rd_tr(sC, u * 32 + 16 * x, L.trc[1][n]), pf[x], oacc[n]);
    }
}

// One wave's part of the walk over the tiles of one (chain, segment).  Wave w = 2rb + ch: units as in
// the header; state blocks: waves 0, 1 the R blocks with kb in {2ch, 2ch + 1}, waves 2, 3 the S blocks
// with kb in {2ch, 2ch + 1} (eight blocks each, all four nb).
__device__ __forceinline__ void bwd1_wave(const Bwd1Args &p, u16 *smem, int chain, int seg, int wave, int lane0) {
    const int rb = wave >> 1, ch = wave & 1;
    const bool s_kind = wave >= 2;   // this wave's state blocks are S (else R)
    const int kb0 = 2 * ch;
    const int tid = threadIdx.x;
    int h = lane0 >> 5, col = lane0 & 31;
    const int64_t T = p.T;
    const int64_t NT = (T + TB1 - 1) / TB1;
    const int64_t tile_lo = (int64_t)seg * p.seg_tiles;
    const int64_t tile_hi = min(tile_lo + p.seg_tiles, NT);
    const int ntiles = (int)(tile_hi - tile_lo);

    const LaneOff L = lane_offsets(lane0, ch);
    const int64_t base = (int64_t)chain * T * D1;
    const u16 *gq = static_cast<const u16 *>(p.q) + base, *gk = static_cast<const u16 *>(p.k) + base;
    const u16 *gv = static_cast<const u16 *>(p.v) + base, *go = static_cast<const u16 *>(p.dout) + base;
    u16 *gdq = static_cast<u16 *>(p.dq) + base, *gdk = static_cast<u16 *>(p.dk) + base,
        *gdv = static_cast<u16 *>(p.dv) + base;
    // R at the segment's end (0 for the last segment), S after the segment's last position
    const float *gR = seg < p.nseg - 1
                          ? p.r_states + ((int64_t)chain * p.r_nsub + state_index(seg, p.r_sub, p.r_nsub, true)) * D1 * D1
                          : nullptr;
    const float *gS = seg < p.nseg - 1 ? p.s_states + ((int64_t)chain * p.s_nsub + (seg + 1) * p.s_sub) * D1 * D1
                                       : p.s_final + (int64_t)chain * D1 * D1;

    f32x16 sacc[8];
    {
        const float *g = s_kind ? gS : gR;
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
    // this wave's blocks as R^T or S^T (bf16, [d_v][d]) into LDS
    auto write_state = [&]() {
        u16 *dst = smem + (s_kind ? oST1 : oRT1);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int nb = s % 4;
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                u32x2 a, c;
                a[0] = pack_bf16(sacc[s][8 * jp + 0], sacc[s][8 * jp + 1]);
                a[1] = pack_bf16(sacc[s][8 * jp + 2], sacc[s][8 * jp + 3]);
                c[0] = pack_bf16(sacc[s][8 * jp + 4], sacc[s][8 * jp + 5]);
                c[1] = pack_bf16(sacc[s][8 * jp + 6], sacc[s][8 * jp + 7]);
                lds_write(dst, nb * 32 * D1 + L.pw[s / 4][jp], join_halves(a, c));
            }
        }
    };

    auto tile_of = [&](int it) -> int64_t { return tile_hi - 1 - it; };
    Staged1 st;
    load_tile1(st, gq, gk, gv, go, tile_of(0) * TB1, T, tid);
    store_tile1(st, smem, tid);
    if (!s_kind) write_state();
    lds_barrier();
    bool r_nonzero = gR != nullptr;

    for (int it = 0; it < ntiles; ++it) {
        const int64_t t0 = tile_of(it) * TB1;
        const bool more = it + 1 < ntiles;
        const int lane = lane0;

        // state updates of this wave's blocks: R += Q^T dO (the old R^T stays in LDS for this tile), or
        // S -= K^T V (the state before this tile) followed by S^T in bf16 for dQ; each operand
        // fragment is read once per 16 positions and shared by the blocks that use it
        {
            const u16 *sA = smem + (s_kind ? oK1 : oQ1), *sC = smem + (s_kind ? oV1 : oO1);
#pragma unroll 1
            for (int x = 0; x < TB1 / 16; ++x) {
                bf16x8 fa[2], fc[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    // this wave's state row blocks kb0 + i are its column blocks 2ch + i
                    fa[i] = rd_tr(sA, 16 * x, L.trc[0][i]);
                    if (s_kind) fa[i] = neg8(fa[i]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) fc[i] = rd_tr(sC, 16 * x, L.trn[i]);
#pragma unroll
                for (int s = 0; s < 8; ++s) sacc[s] = mfma(fa[s / 4], fc[s % 4], sacc[s]);
            }
        }
        if (s_kind) write_state();
        // the next tile's inputs: in flight while this tile's three gradients are formed
        if (more) load_tile1(st, gq, gk, gv, go, tile_of(it + 1) * TB1, T, tid);

        // Each unit is staged in this wave's own 8 KiB of LDS and stored as whole 128-byte row pieces
        // as soon as it is done, so that at most one unit's accumulators are held at a time.
        u16 *ob = smem + oOS1 + wave * kOS1;
        auto stage = [&](const f32x16 (&acc)[2], u16 *dst) {
            // 16 lanes writing one chunk of 16 consecutive rows (or reading whole rows) hit 16 bank groups
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    u32x2 a, c;
                    a[0] = pack_bf16(acc[n][8 * jp + 0], acc[n][8 * jp + 1]);
                    a[1] = pack_bf16(acc[n][8 * jp + 2], acc[n][8 * jp + 3]);
                    c[0] = pack_bf16(acc[n][8 * jp + 4], acc[n][8 * jp + 5]);
                    c[1] = pack_bf16(acc[n][8 * jp + 6], acc[n][8 * jp + 7]);
                    const int chk = 4 * n + 2 * jp + h;
                    lds_write(dst, col * 64 + ((chk ^ ((col >> 1) & 7)) << 3), join_halves(a, c));
                }
        };
        auto store = [&](const u16 *src, u16 *g, int orow) {
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(g + t0 * D1, (T - t0) * D1 * 2);
            u32x4 v[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int qd = lane + 64 * s2, row = qd / 8, chk = qd % 8;
                v[s2] = *reinterpret_cast<const u32x4 *>(src + row * 64 + ((chk ^ ((row >> 1) & 7)) << 3));
            }
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int qd = lane + 64 * s2, row = qd / 8, chk = qd % 8;
                bstore16(ry, ((orow * 32 + row) * D1 + ch * 64 + chk * 8) * 2, v[s2]);
            }
        };
        {
            f32x16 oacc[2];
            out_unit<Unit::DV>(oacc, smem, rb, ch, lane, L, r_nonzero);
            stage(oacc, ob);
            out_unit<Unit::DK>(oacc, smem, rb, ch, lane, L, r_nonzero);
            stage(oacc, ob + 2048);
            store(ob, gdv, rb);
            store(ob + 2048, gdk, rb);
        }
        lds_barrier();   // S^T of the state before this tile is complete
        {
            f32x16 oacc[2];
            out_unit<Unit::DQ>(oacc, smem, 1 - rb, ch, lane, L, true);
            stage(oacc, ob);
            store(ob, gdq, 1 - rb);
        }
        lds_barrier();   // every wave is done with this tile's inputs, R^T and S^T
        if (!s_kind) write_state();
        r_nonzero = true;
        if (more) store_tile1(st, smem, tid);
        lds_barrier();
    }
}

__global__ __launch_bounds__(kT1, 1) void bwd1_bf16_kernel(Bwd1Args p) {
    __shared__ __attribute__((aligned(16))) u16 smem[kLds1];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int seg = blockIdx.x % p.nseg;
    const int chain = blockIdx.x / p.nseg;
    const int64_t NT = (p.T + TB1 - 1) / TB1;
    if ((int64_t)seg * p.seg_tiles >= NT) return;
    bwd1_wave(p, smem, chain, seg, wave, lane);
}

}  // namespace

hipError_t launch_bwd1_bf16(const Bwd1Args &a, hipStream_t s) {
    const unsigned items = (unsigned)((int64_t)a.chains * a.nseg);
    hipLaunchKernelGGL(bwd1_bf16_kernel, dim3(items), dim3(kT1), 0, s, a);
    return hipGetLastError();
}

}  // namespace la2
