// la2_scan_bf16.hip -- bf16 tile-scan kernel of Lightning Attention-2 on gfx950 MFMA.
//
// One workgroup (8 waves, two per SIMD) owns one (chain, segment, value-slice) work item and walks
// the segment's tiles in order (page "Lightning Attention", lizeman.github.io llm-arch-kb,
// section 2, Steps 1-4).  Per tile of TB positions it computes
//
//   A^T   = K_b Q_b^T                 (Step 2 scores, transposed, fp32 in MFMA accumulators)
//   P     = causal decay mask of A    (kept in registers; becomes the next MFMA's A operand)
//   O_b^T = S^T Q_b^T diag(w_inter) + V_b^T P^T   (Step 3 right + Step 2 left product, as O^T)
//   S     = lam^TB S + (diag(w_upd) K_b)^T V_b   (Step 4, fp32 accumulators, never leaves chip)
//
// with the decay weights of the token recurrence S_t = lam S_{t-1} + k_t v_t^T:
//   forward: mask lam^(i-j) for j <= i, w_inter = lam^(i+1),  w_upd = lam^(TB-1-j)
//   reverse: mask lam^(j-i) for j >= i, w_inter = lam^(TB-i), w_upd = lam^j
// The reverse direction is the same scan run from the last tile to the first; the backward pass
// uses it for dK and dV.  All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// LDS holds the tiles in their natural row-major layout, rows split in 16-byte chunks whose
// position is XOR-swizzled by row:
//   sQ  [TB][D]   Q tile      (A^T B operand and Q S A operand: plain 16-byte fragment reads)
//   sK  [TB][D]   K tile      (A^T A operand: plain reads; state-update A operand K^T: transpose reads)
//   sV  [TB][DV]  V tile      (P V and state-update B operand V: transpose reads)
//   sST [DV][D]   S^T in bf16 (Q S B operand)
//   sKW [TB][D]   K rows weighted by w_upd (decay only: the state update's A operand)
//   sOS           per-wave output staging (where LDS allows; with decay at TB = 128, sKW once the
//                 state update is done with it)
// Operands that need 8 consecutive positions per lane (K^T, V) come from ds_read_b64_tr_b16: in
// each group of 16 lanes, lane i receives element i%4 of the 8-byte rows addressed by lanes
// i/4 + 4e, so lanes that address (row R0 + j/4, column C0 + 4 (j%4)) get column C0 + i, rows
// R0..R0+3.  Where two tile buffers fit in LDS the next tile goes global -> LDS directly, one whole
// tile ahead; otherwise it is staged global -> registers -> LDS, its loads issued during the
// current tile (without decay the query-role tile at its top, the others after the intra-tile
// phase).  Output tiles are staged per wave in LDS and stored as whole rows; with the normalized
// form each output row is divided by its denominator first.
#include "la2_bf16_common.h"

namespace la2 {
namespace {

using namespace dev;

template <int D, int DV, int TB, bool DECAY = false>
struct Cfg {
    static constexpr int NTB = TB / 32;          // 32-row blocks of the tile
    static constexpr int NDB = DV / 32;          // 32-column blocks of the value slice
    static constexpr int NKB = D / 32;           // 32-row blocks of the state
    static constexpr int WPT = (kWaves / NTB < NDB) ? kWaves / NTB : NDB;   // waves sharing one row block
    static constexpr int ODB = NDB / WPT;        // value blocks of O per wave
    static constexpr int NSB = NKB * NDB;        // 32x32 blocks of the state
    static constexpr int SPW = NSB > kWaves ? NSB / kWaves : 1;   // state blocks per wave
    static constexpr int KS = D / 16;            // contraction steps over d
    // global -> register staging, 16-byte chunks of the natural tiles
    static constexpr int QCH = TB * D / 8;
    static constexpr int KCH = TB * D / 8;
    static constexpr int VCH = TB * DV / 8;
    static constexpr int NQ = (QCH + kThreads - 1) / kThreads;
    static constexpr int NK = (KCH + kThreads - 1) / kThreads;
    static constexpr int NV = (VCH + kThreads - 1) / kThreads;
    // LDS carve-up (bf16 elements).  A tile buffer holds Q, K and V; there are two of them, filled
    // by direct global -> LDS loads one tile ahead, when they fit (kDMA), else one, filled from
    // registers.
    static constexpr int TILE = TB * D + TB * D + TB * DV;
    static constexpr int oQ = 0;                             // offsets inside a tile buffer
    static constexpr int oK = oQ + TB * D;
    static constexpr int oV = oK + TB * D;
    // per-wave staging of its 32 x ODB*32 output block, for full-row stores: in a region of its own
    // where LDS allows (kStageO), else (decay) in the weighted K copy once the state update is done
    // with it (kStageLate), O waiting in registers until then
    static constexpr int OSW = ODB * 32;                     // staged row width (elements)
    static constexpr int OSZ = kWaves * 32 * OSW;
    static constexpr int KWZ = DECAY ? TB * D : 0;           // weighted K copy
    static constexpr bool fits(int nbuf, bool own_os) {
        return (nbuf * TILE + DV * D + KWZ + (own_os ? OSZ : 0)) * 2 <= 160 * 1024;
    }
    static constexpr bool kLateOK = DECAY && OSZ <= KWZ;
    static constexpr bool kDMA = fits(2, true) || (kLateOK && fits(2, false));
    static constexpr int NBUF = kDMA ? 2 : 1;
    static constexpr bool kStageO = fits(NBUF, true);
    static constexpr bool kStageLate = !kStageO;
    static constexpr int oST = NBUF * TILE;                  // S^T in bf16
    static constexpr int oKW = oST + DV * D;                 // K rows weighted by w_upd (decay only)
    static constexpr int oOS = oKW + KWZ;
    static constexpr int kLds = oOS + (kStageO ? OSZ : 0);
    static_assert(NTB == 2 || NTB == 4, "tile of 64 or 128 positions");
    static_assert(ODB * WPT == NDB && NTB * WPT <= kWaves, "output blocks");
    static_assert(SPW * kWaves == NSB || (SPW == 1 && NSB <= kWaves), "state blocks");
    static_assert(kLds * 2 <= 160 * 1024, "LDS");
    static_assert(!kStageLate || kLateOK, "late output staging fits the K copy");
};

// Row block and part (which ODB value blocks) of O owned by a wave.  Waves w and w + 4 share a
// SIMD; the mapping gives each SIMD one short and one long causal row block.
template <int NTB, int WPT>
__device__ __forceinline__ void wave_rows(int wave, int &tb, int &part) {
    if constexpr (NTB == 4 && WPT == 2) {
        tb = wave < 4 ? wave : 7 - wave;
        part = wave < 4 ? 0 : 1;
    } else if constexpr (NTB == 2 && WPT == 4) {
        tb = (wave & 1) ^ ((wave >> 2) & 1);
        part = (wave >> 1) & 3;
    } else {
        tb = wave % NTB;
        part = wave / NTB;
    }
}

template <int D, int DV, int TB>
struct Staged {
    using C = Cfg<D, DV, TB>;
    u32x4 q[C::NQ];
    u32x4 k[C::NK];
    u32x4 v[C::NV];
};

// Issue the global loads of the tile starting at position t0 into registers (16-byte chunks of
// the natural row-major tiles).  Nothing waits for them here; rows at or past T read as zero.
// PART: 0 all three tiles, 1 the query-role tile only, 2 the key- and value-role tiles only.
template <int D, int DV, int TB, int PART = 0>
__device__ __forceinline__ void stage_load(Staged<D, DV, TB> &r, const u16 *a, const u16 *b, const u16 *c,
                                           int64_t t0, int64_t T, int DVT, int tid) {
    using C = Cfg<D, DV, TB>;
    if constexpr (PART != 2) {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a + t0 * D, (T - t0) * D * 2);
#pragma unroll
        for (int s = 0; s < C::NQ; ++s) {
            const int cid = min(tid + s * kThreads, C::QCH - 1);
            r.q[s] = bload(ra, ((cid / (D / 8)) * D + (cid % (D / 8)) * 8) * 2);
        }
    }
    if constexpr (PART == 1) return;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b + t0 * D, (T - t0) * D * 2);
#pragma unroll
    for (int s = 0; s < C::NK; ++s) {
        const int cid = min(tid + s * kThreads, C::KCH - 1);
        r.k[s] = bload(rb, ((cid / (D / 8)) * D + (cid % (D / 8)) * 8) * 2);
    }
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(c + t0 * DVT, (T - t0) * DVT * 2);
#pragma unroll
    for (int s = 0; s < C::NV; ++s) {
        const int cid = min(tid + s * kThreads, C::VCH - 1);
        r.v[s] = bload(rc, ((cid / (DV / 8)) * DVT + (cid % (DV / 8)) * 8) * 2);
    }
}

template <int D, int DV, int TB, Dir DIR, bool DECAY>
__device__ __forceinline__ void stage_store(const Staged<D, DV, TB> &r, u16 *smem, int tid, float l2) {
    using C = Cfg<D, DV, TB, DECAY>;
#pragma unroll
    for (int s = 0; s < C::NQ; ++s) {
        const int cid = tid + s * kThreads;
        if (cid < C::QCH) lds_write(smem + C::oQ, nat_off<D>(cid / (D / 8), cid % (D / 8)), r.q[s]);
    }
#pragma unroll
    for (int s = 0; s < C::NK; ++s) {
        const int cid = tid + s * kThreads;
        if (cid < C::KCH) {
            const int row = cid / (D / 8), off = nat_off<D>(row, cid % (D / 8));
            lds_write(smem + C::oK, off, r.k[s]);
            if constexpr (DECAY) {
                // the state update's copy of K: row j scaled by w_upd(j), rounded once to bf16
                const float w = __builtin_amdgcn_exp2f((float)(DIR == Dir::Forward ? TB - 1 - row : row) * l2);
                u32x4 x = r.k[s];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    x[m] = f32_to_bf16(__uint_as_float(x[m] << 16) * w) |
                           (f32_to_bf16(__uint_as_float(x[m] & 0xffff0000u) * w) << 16);
                lds_write(smem + C::oKW, off, x);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < C::NV; ++s) {
        const int cid = tid + s * kThreads;
        if (cid < C::VCH) lds_write(smem + C::oV, nat_off<DV>(cid / (DV / 8), cid % (DV / 8)), r.v[s]);
    }
}

// Issue the direct loads of the tile starting at position t0 into the tile buffer at `buf`.
template <int D, int DV, int TB>
__device__ __forceinline__ void dma_tile(u16 *buf, const u16 *a, const u16 *b, const u16 *c, int64_t t0, int64_t T,
                                         int DVT, int wave, int lane) {
    using C = Cfg<D, DV, TB>;
    dma_rows<D, TB>(make_rsrc(a + t0 * D, (T - t0) * D * 2), buf + C::oQ, D, wave, lane);
    dma_rows<D, TB>(make_rsrc(b + t0 * D, (T - t0) * D * 2), buf + C::oK, D, wave, lane);
    dma_rows<DV, TB>(make_rsrc(c + t0 * DVT, (T - t0) * DVT * 2), buf + C::oV, DVT, wave, lane);
}

template <int D, int DV, int TB, Dir DIR, bool DECAY, bool NORM>
__global__ __launch_bounds__(kThreads, 1) void scan_bf16_kernel(ScanArgs p) {
    using C = Cfg<D, DV, TB, DECAY>;
    __shared__ __attribute__((aligned(16))) u16 smem[C::kLds];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;

    // work item; workgroups are dealt to the 8 XCDs round robin, so when the grid allows, the
    // slices of one (chain, segment) get block ids that land on the same XCD and share its L2
    int item = blockIdx.x;
    if (p.nslice > 1 && gridDim.x % (8 * p.nslice) == 0) {
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

    const u16 *ga = static_cast<const u16 *>(p.a) + (int64_t)chain * T * D;
    const u16 *gb = static_cast<const u16 *>(p.b) + (int64_t)chain * T * D;
    const u16 *gc = static_cast<const u16 *>(p.c) + (int64_t)chain * T * p.DVT + dv0;
    u16 *gy = static_cast<u16 *>(p.y) + (int64_t)chain * T * p.DVT + dv0;
    const int sidx = state_index(seg, p.sub, p.nsub, DIR == Dir::Reverse);
    float *gs = p.states ? p.states + ((int64_t)chain * p.nsub + sidx) * D * p.DVT + (p.states_t ? (int64_t)dv0 * D : dv0)
                         : nullptr;

    // lam^n = 2^(n log2 lam) with the hardware exp2 (n >= 0 only, so no overflow; tiny powers flush to 0)
    const float l2 = DECAY ? log2f(p.decay[chain % p.H]) : 0.0f;
    auto pw = [&](int n) -> float { return DECAY ? __builtin_amdgcn_exp2f((float)n * l2) : 1.0f; };

    // waves -> blocks of O (row block tb, value blocks db0 .. db0 + ODB - 1) and of the state
    int tb, part;
    wave_rows<C::NTB, C::WPT>(wave, tb, part);
    const bool o_active = part < C::WPT;
    const int db0 = part * C::ODB;
    const bool s_active = wave * C::SPW < C::NSB;

    f32x16 sacc[C::SPW];
    const bool init_state = gs != nullptr &&
                            (DIR == Dir::Forward ? (seg > 0 || p.has_init) : (seg < p.nseg - 1 || p.has_init));
    // A reverse output pass with a carried-in state (the gradient of a carried-out forward state)
    // has it attached at the chain's last position: on the chain's last tile, the first this
    // workgroup processes, its rows are weighted lam^(leff-1-i) and it is carried on with
    // lam^(leff-1), leff the tile's real length.
    const bool end_init = DIR == Dir::Reverse && p.has_init && seg == p.nseg - 1;
    const int leff_end = (int)min((int64_t)TB, T - (NT - 1) * TB);
#pragma unroll
    for (int s = 0; s < C::SPW; ++s) {
        const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const int64_t e = p.states_t ? (int64_t)(nb * 32 + col) * D + d : (int64_t)d * p.DVT + nb * 32 + col;
            sacc[s][r] = (init_state && s_active) ? gs[e] : 0.0f;
        }
    }

    auto tile_of = [&](int it) -> int64_t { return DIR == Dir::Forward ? tile_lo + it : tile_hi - 1 - it; };

    // S^T (bf16) into LDS for the next tile's right product
    auto write_state_lds = [&]() {
        if (!s_active) return;
#pragma unroll
        for (int s = 0; s < C::SPW; ++s) {
            const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
            // lane (col, h) holds d = kb*32 + 8j + 4h + 0..3 of row nb*32 + col: pair up the two
            // halves of chunks j and j + 1 across h, so every lane writes one whole 16-byte chunk
            // (8-byte writes of one half would leave half the banks idle: 2-way conflicts)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                u32x2 a, b;
                a[0] = pack_bf16(sacc[s][8 * jp + 0], sacc[s][8 * jp + 1]);
                a[1] = pack_bf16(sacc[s][8 * jp + 2], sacc[s][8 * jp + 3]);
                b[0] = pack_bf16(sacc[s][8 * jp + 4], sacc[s][8 * jp + 5]);
                b[1] = pack_bf16(sacc[s][8 * jp + 6], sacc[s][8 * jp + 7]);
                const u32x4 w = join_halves(a, b);
                lds_write(smem + C::oST, nat_off<D>(nb * 32 + col, kb * 4 + 2 * jp + h), w);
            }
        }
    };

    Staged<D, DV, TB> st;
    if constexpr (C::kDMA) {
        dma_tile<D, DV, TB>(smem, ga, gb, gc, tile_of(0) * TB, T, p.DVT, wave, lane);
        wait_vm();
        lds_barrier();
        if constexpr (DECAY) build_kw<D, TB, DIR>(smem + C::oK, smem + C::oKW, tid, l2, 0);
    } else {
        stage_load<D, DV, TB>(st, ga, gb, gc, tile_of(0) * TB, T, p.DVT, tid);
        stage_store<D, DV, TB, DIR, DECAY>(st, smem, tid, l2);
    }
    if (init_state) write_state_lds();
    lds_barrier();

    const u16 *sST = smem + C::oST;
    bool state_nonzero = init_state;
    int it = 0;
    // One tile: `cur` is the tile buffer it reads, `nxt` the one the next tile's direct loads fill.
    auto tile = [&](const u16 *cur, u16 *nxt) __attribute__((always_inline)) {
        const int64_t t0 = tile_of(it) * TB;
        const bool update = it + 1 < ntiles;
        const u16 *sQ = cur + C::oQ, *sK = cur + C::oK, *sV = cur + C::oV;
        // the next tile's direct loads go out first and have this whole tile to land; its buffer was
        // last read in the previous tile, which every wave has left
        if constexpr (C::kDMA) {
            if (it + 1 < ntiles) dma_tile<D, DV, TB>(nxt, ga, gb, gc, tile_of(it + 1) * TB, T, p.DVT, wave, lane);
        } else if constexpr (!DECAY) {
            // register staging: the next query-role tile (16 VGPRs) goes out now and has the whole tile
            // to land; its key and value tiles follow after the intra-tile phase (measured ~1.5%
            // faster without decay; with decay, where registers are scarcer, all three go out later)
            if (it + 1 < ntiles) stage_load<D, DV, TB, 1>(st, ga, gb, gc, tile_of(it + 1) * TB, T, p.DVT, tid);
        }

        // O^T accumulators of this wave's output block, and their store: each lane holds 4
        // consecutive columns of its row tb*32 + col per group; rows at or past T fall outside the
        // buffer range and are dropped.  Through a private LDS block at `ob`: 8-byte writes of the
        // O^T groups, then 16-byte reads of whole rows, so every store instruction writes 8 full
        // 128-byte rows.
        f32x16 oacc[C::ODB];
        // normalized form: the denominator of this lane's row, fetched now so that its load has the
        // tile to land (rows past T divide by 1 and are not stored)
        float den = 1.0f;
        if constexpr (NORM) {
            const int64_t t = t0 + tb * 32 + col;
            if (t < T) den = p.den[(int64_t)chain * T + t];
        }
        auto store_o = [&](u16 *ob) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(gy + t0 * p.DVT, (T - t0) * p.DVT * 2);
            if constexpr (NORM) {
                const float rd = 1.0f / den;
#pragma unroll
                for (int n = 0; n < C::ODB; ++n) oacc[n] *= rd;
            }
            constexpr int NC = C::OSW / 8;   // 16-byte chunks per staged row
            // chunk swizzle: 16 lanes writing one chunk of 16 consecutive rows (or reading whole rows)
            // touch 16 different bank groups
            auto oswz = [&](int row) { return (row / (16 / NC)) & (NC - 1); };
#pragma unroll
            for (int n = 0; n < C::ODB; ++n)
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    // lane (col, h) holds columns n*32 + 8j + 4h + 0..3: pair the halves of chunks
                    // j = 2jp and 2jp + 1 across h and write whole chunks
                    u32x2 a, b;
                    a[0] = pack_bf16(oacc[n][8 * jp + 0], oacc[n][8 * jp + 1]);
                    a[1] = pack_bf16(oacc[n][8 * jp + 2], oacc[n][8 * jp + 3]);
                    b[0] = pack_bf16(oacc[n][8 * jp + 4], oacc[n][8 * jp + 5]);
                    b[1] = pack_bf16(oacc[n][8 * jp + 6], oacc[n][8 * jp + 7]);
                    const u32x4 w = join_halves(a, b);
                    const int ch = 4 * n + 2 * jp + h;
                    lds_write(ob, col * C::OSW + ((ch ^ oswz(col)) << 3), w);
                }
#pragma unroll
            for (int s2 = 0; s2 < 32 * NC / 64; ++s2) {
                const int q = lane + 64 * s2, row = q / NC, ch = q % NC;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + row * C::OSW + ((ch ^ oswz(row)) << 3));
                bstore16(ry, ((tb * 32 + row) * p.DVT + db0 * 32 + ch * 8) * 2, v);
            }
        };

        if (o_active) {
            const int qrow = tb * 32 + col;
            auto rdQ = [&](int ks) { return lds_read(sQ, nat_off<D>(qrow, 2 * ks + h)); };

#pragma unroll
            for (int n = 0; n < C::ODB; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0f;

            // Step 3: inter-tile right product, rows weighted by w_inter
            if (state_nonzero) {
                auto rdST = [&](int n, int ks) {
                    return lds_read(sST, nat_off<D>((db0 + n) * 32 + col, 2 * ks + h));
                };
                bf16x8 qa = rdQ(0), sa[C::ODB];
#pragma unroll
                for (int n = 0; n < C::ODB; ++n) sa[n] = rdST(n, 0);
#pragma unroll 2
                for (int ks = 0; ks < C::KS; ++ks) {
                    const int kn = ks + 1 < C::KS ? ks + 1 : ks;
                    const bf16x8 qn = rdQ(kn);
                    bf16x8 sn[C::ODB];
#pragma unroll
                    for (int n = 0; n < C::ODB; ++n) sn[n] = rdST(n, kn);
#pragma unroll
                    for (int n = 0; n < C::ODB; ++n) oacc[n] = mfma(sa[n], qa, oacc[n]);
                    qa = qn;
#pragma unroll
                    for (int n = 0; n < C::ODB; ++n) sa[n] = sn[n];
                }
                if constexpr (DECAY) {
                    // every accumulator of this lane belongs to the row tb*32 + col
                    const int i = tb * 32 + col;
                    int e = DIR == Dir::Forward ? i + 1 : TB - i;
                    if (DIR == Dir::Reverse && end_init && it == 0) e = leff_end - 1 - i;
                    const float w = e >= 0 ? pw(e) : 0.0f;
#pragma unroll
                    for (int n = 0; n < C::ODB; ++n)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[n][r] *= w;
                }
            }

            // Step 2: intra-tile masked left product, one 32x32 block of A^T at a time
            const int ulo = DIR == Dir::Forward ? 0 : tb;
            const int uhi = DIR == Dir::Forward ? tb : C::NTB - 1;
            const int tcol = tb * 32 + col;
            for (int u = ulo; u <= uhi; ++u) {
                asm volatile("" ::: "memory");   // keep each block's LDS reads inside its iteration
                // V fragments of this block, in P's row order; in the forward direction they are read
                // before the A^T chain, which hides their latency
                bf16x8 vf[2][C::ODB];
                auto rdVF = [&](int x, int n) { return frag_tr<DV, true>(sV, u * 32 + 16 * x, (db0 + n) * 32, lane); };
                if constexpr (DIR == Dir::Forward) {
#pragma unroll
                    for (int x = 0; x < 2; ++x)
#pragma unroll
                        for (int n = 0; n < C::ODB; ++n) vf[x][n] = rdVF(x, n);
                }
                f32x16 acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
                bf16x8 ka = lds_read(sK, nat_off<D>(u * 32 + col, h)), qa = rdQ(0);
#pragma unroll
                for (int ks = 0; ks < C::KS; ks += 2) {
                    const bf16x8 kb = lds_read(sK, nat_off<D>(u * 32 + col, 2 * (ks + 1) + h)), qb = rdQ(ks + 1);
                    acc = mfma(ka, qa, acc);
                    if (ks + 2 < C::KS) {
                        ka = lds_read(sK, nat_off<D>(u * 32 + col, 2 * (ks + 2) + h));
                        qa = rdQ(ks + 2);
                    }
                    acc = mfma(kb, qb, acc);
                }
                // causal decay mask: only the diagonal block has masked entries.  The distance of
                // accumulator r is base -/+ (8 (r / 4) + r % 4), small integers exact in fp32; the
                // base is hidden from loop-invariant hoisting, which would otherwise keep the
                // per-lane distances or weights across the tile loop in spilled registers (and
                // every spill reload waits on the next tile's loads).
                float base = (float)(DIR == Dir::Forward ? tcol - u * 32 - 4 * h : u * 32 + 4 * h - tcol);
                asm volatile("" : "+v"(base));
                bf16x8 pf[2];
                if (DECAY && u != tb) {
                    // off the diagonal every distance is >= 1: one exp per group of 4 accumulators,
                    // lam^dist = lam^(smallest distance in the group) * lam^(offset from it), both
                    // exponents >= 0, so neither factor can overflow (lam^e is rebuilt per block from
                    // a hidden copy of log2 lam rather than held across the tile loop)
                    float l2b = l2;
                    asm volatile("" : "+v"(l2b));
                    const float lam_e[4] = {1.0f, __builtin_amdgcn_exp2f(l2b), __builtin_amdgcn_exp2f(2.0f * l2b),
                                            __builtin_amdgcn_exp2f(3.0f * l2b)};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float pm = __builtin_amdgcn_exp2f(
                            (DIR == Dir::Forward ? base - (float)(8 * m + 3) : base + (float)(8 * m)) * l2);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * m + e;
                            pf[r >> 3][r & 7] = (__bf16)(acc[r] * (pm * lam_e[DIR == Dir::Forward ? 3 - e : e]));
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float c = (float)(8 * (r >> 2) + (r & 3));
                        const float diff = DIR == Dir::Forward ? base - c : base + c;
                        const float w = DECAY ? __builtin_amdgcn_exp2f(diff * l2) : 1.0f;
                        const float v = diff >= 0.0f ? (DECAY ? acc[r] * w : acc[r]) : 0.0f;
                        pf[r >> 3][r & 7] = (__bf16)v;
                    }
                }
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int n = 0; n < C::ODB; ++n)
                        oacc[n] = mfma(DIR == Dir::Forward ? vf[x][n] : rdVF(x, n), pf[x], oacc[n]);
            }

            // with the LDS to spare, O goes out now; otherwise (decay: the weighted K copy fills
            // LDS) it waits in registers until the state update has released that copy
            if constexpr (C::kStageO) store_o(smem + C::oOS + wave * 32 * C::OSW);
        }

        // Without the second buffer, the next tile's loads (all, or the key and value tiles) go out
        // here, after the register-heavy intra-tile phase, and land in LDS after this tile's last
        // barrier.
        if constexpr (!C::kDMA) {
            if (it + 1 < ntiles)
                stage_load<D, DV, TB, DECAY ? 0 : 2>(st, ga, gb, gc, tile_of(it + 1) * TB, T, p.DVT, tid);
        }

        // Step 4: state update S = lam^TB S + (w_upd K)^T V, fp32 accumulators
        if (update) {
            if (s_active) {
                if constexpr (DECAY) {
                    const float f = (DIR == Dir::Reverse && end_init && it == 0) ? pw(leff_end - 1) : pw(TB);
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) sacc[s] *= f;
                }
                const u16 *sKU = DECAY ? smem + C::oKW : sK;   // K as used by the update
                // with O held in registers across the update, its fragment addresses are rebuilt here
                // from a hidden copy of the lane index rather than kept (and spilled) across the loop
                int ln = lane;
                if constexpr (C::kStageLate) asm volatile("" : "+v"(ln));
                auto rdKT = [&](int s, int x) {
                    return frag_tr<D, false>(sKU, 16 * x, ((wave * C::SPW + s) / C::NDB) * 32, ln);
                };
                auto rdV = [&](int s, int x) {
                    return frag_tr<DV, false>(sV, 16 * x, ((wave * C::SPW + s) % C::NDB) * 32, ln);
                };
                bf16x8 ka[C::SPW], va[C::SPW];
#pragma unroll
                for (int s = 0; s < C::SPW; ++s) {
                    ka[s] = rdKT(s, 0);
                    va[s] = rdV(s, 0);
                }
#pragma unroll 2
                for (int x = 0; x < TB / 16; ++x) {
                    bf16x8 kn[C::SPW], vn[C::SPW];
                    const int xn = x + 1 < TB / 16 ? x + 1 : x;
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) {
                        kn[s] = rdKT(s, xn);
                        vn[s] = rdV(s, xn);
                    }
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) sacc[s] = mfma(ka[s], va[s], sacc[s]);
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) {
                        ka[s] = kn[s];
                        va[s] = vn[s];
                    }
                }
            }
            state_nonzero = true;
        }

        if constexpr (C::kDMA) {
            wait_vm();                       // this wave's loads of the next tile have landed
            lds_barrier();                   // ... everyone's, and every wave is done with this tile
            if (update) write_state_lds();
            if constexpr (C::kStageLate) {
                if (o_active) store_o(smem + C::oKW + wave * 32 * C::OSW);
                lds_barrier();               // every staged O is read back before the copy is rebuilt
            }
            if constexpr (DECAY) {
                if (it + 1 < ntiles)
                    build_kw<D, TB, DIR>(nxt + C::oK, smem + C::oKW, tid, l2);
            }
        } else {
            lds_barrier();                   // every wave is done with this tile's LDS
            if (update) write_state_lds();
            if constexpr (C::kStageLate) {
                if (o_active) store_o(smem + C::oKW + wave * 32 * C::OSW);
                lds_barrier();               // every staged O is read back before the copy is rebuilt
            }
            if (it + 1 < ntiles) stage_store<D, DV, TB, DIR, DECAY>(st, smem, tid, l2);
        }
        lds_barrier();
    };
    for (; it < ntiles; ++it) {
        if constexpr (C::kDMA) {
            // The two buffers are distinct and nothing else in a tile touches them, which the
            // restrict qualifiers state; without that the compiler makes every LDS transpose read
            // wait for the next tile's loads.
            [&](const u16 *__restrict__ cur, u16 *__restrict__ nxt) __attribute__((always_inline)) {
                tile(cur, nxt);
            }(smem + (it & 1) * C::TILE, smem + ((it + 1) & 1) * C::TILE);
        } else {
            tile(smem, smem);
        }
    }

    // Carried-out state, from the workgroup that processes the chain's last tile in scan order.
    // Forward: the final state, i.e. the last tile's update (which the loop leaves out) over its
    // `leff` real positions, S = lam^leff S + sum_{j < leff} lam^(leff-1-j) k_j v_j^T (exact for a
    // ragged last tile).  Reverse: lam times the state at position 0, R = lam^TB R + sum_j lam^j
    // b_j c_j^T over tile 0 (rows past T are zero) -- the gradient of a carried-in forward state.
    // The last tile is still in LDS and nothing writes LDS any more; its weights are applied to the
    // fragments in registers (the weighted copy may hold staged outputs by now).
    const bool want = p.state_out != nullptr && s_active && (DIR == Dir::Forward ? seg == p.nseg - 1 : seg == 0);
    if (want) {
        const int last = ntiles - 1;
        const u16 *cur = smem + (C::kDMA ? (last & 1) * C::TILE : 0);
        const u16 *sK = cur + C::oK, *sV = cur + C::oV;
        const int leff = (int)min((int64_t)TB, T - tile_of(last) * TB);
        if constexpr (DECAY) {
            const float f = DIR == Dir::Forward ? pw(leff) : (end_init && ntiles == 1 ? pw(leff_end - 1) : pw(TB));
#pragma unroll
            for (int s = 0; s < C::SPW; ++s) sacc[s] *= f;
        }
#pragma unroll
        for (int s = 0; s < C::SPW; ++s) {
            const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
            for (int x = 0; x < TB / 16; ++x) {
                bf16x8 kf = frag_tr<D, false>(sK, 16 * x, kb * 32, lane);
                if constexpr (DECAY) {
                    // rows j = 16x + 8h + e: forward lam^(leff-1-j) and 0 past the sequence end,
                    // reverse lam^j
                    u32x4 u = __builtin_bit_cast(u32x4, kf);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int j = 16 * x + 8 * h + 2 * m;
                        float wl, wh;
                        if constexpr (DIR == Dir::Forward) {
                            wl = j < leff ? __builtin_amdgcn_exp2f((float)(leff - 1 - j) * l2) : 0.0f;
                            wh = j + 1 < leff ? __builtin_amdgcn_exp2f((float)(leff - 2 - j) * l2) : 0.0f;
                        } else {
                            wl = __builtin_amdgcn_exp2f((float)j * l2);
                            wh = __builtin_amdgcn_exp2f((float)(j + 1) * l2);
                        }
                        u[m] = pack_bf16(__uint_as_float(u[m] << 16) * wl, __uint_as_float(u[m] & 0xffff0000u) * wh);
                    }
                    kf = __builtin_bit_cast(bf16x8, u);
                }
                sacc[s] = mfma(kf, frag_tr<DV, false>(sV, 16 * x, nb * 32, lane), sacc[s]);
            }
            const float scale = DIR == Dir::Reverse ? pw(1) : 1.0f;
            float *so = p.state_out + (int64_t)chain * D * p.DVT + dv0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                so[(int64_t)d * p.DVT + nb * 32 + col] = sacc[s][r] * scale;
            }
        }
    }
}

template <int D, int DV, int TB, Dir DIR, bool NORM>
hipError_t launch_norm(const ScanArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)a.chains * a.seg_count * a.nslice;
    if (a.decay)
        hipLaunchKernelGGL((scan_bf16_kernel<D, DV, TB, DIR, true, NORM>), dim3((unsigned)items), dim3(kThreads), 0, s,
                           a);
    else
        hipLaunchKernelGGL((scan_bf16_kernel<D, DV, TB, DIR, false, NORM>), dim3((unsigned)items), dim3(kThreads), 0,
                           s, a);
    return hipGetLastError();
}

template <int D, int DV, int TB, Dir DIR>
hipError_t launch_one(const ScanArgs &a, hipStream_t s) {
    if constexpr (DIR == Dir::Forward) {
        if (a.den) return launch_norm<D, DV, TB, DIR, true>(a, s);
    } else {
        if (a.den) return hipErrorInvalidValue;
    }
    return launch_norm<D, DV, TB, DIR, false>(a, s);
}

template <int D, int DV>
hipError_t launch_tb(const ScanArgs &a, int TB, Dir dir, hipStream_t s) {
    if (dir == Dir::Forward)
        return TB == 64 ? launch_one<D, DV, 64, Dir::Forward>(a, s) : launch_one<D, DV, 128, Dir::Forward>(a, s);
    return TB == 64 ? launch_one<D, DV, 64, Dir::Reverse>(a, s) : launch_one<D, DV, 128, Dir::Reverse>(a, s);
}

}  // namespace

bool bf16_supported(int D, int DV, int TB) {
    return (D == 64 || D == 128) && (DV == 64 || DV == 128) && (TB == 64 || TB == 128);
}

hipError_t launch_scan_bf16(const ScanArgs &a, int D, int DV, int TB, Dir dir, hipStream_t s) {
    if (!bf16_supported(D, DV, TB)) return hipErrorInvalidValue;
    if (D == 64) return DV == 64 ? launch_tb<64, 64>(a, TB, dir, s) : launch_tb<64, 128>(a, TB, dir, s);
    return DV == 64 ? launch_tb<128, 64>(a, TB, dir, s) : launch_tb<128, 128>(a, TB, dir, s);
}

}  // namespace la2
