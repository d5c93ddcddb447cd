// la2_scan_bf16.hip -- bf16 tile-scan kernel of Lightning Attention-2 on gfx950 MFMA.
//
// One workgroup (8 waves, two per SIMD) owns one (chain, segment, value-slice) work item and walks
// the segment's tiles in order (page "Lightning Attention", lizeman.github.io
// llm-arch-kb, section 2, Steps 1-4).  Per tile of TB positions it computes
//
//   A^T   = K_b Q_b^T                 (Step 2 scores, transposed, fp32 in MFMA accumulators)
//   P     = causal decay mask of A    (kept in registers; becomes the next MFMA's A operand)
//   O_b   = diag(w_inter) Q_b S + P V_b   (Step 3 right product plus Step 2 left product)
//   S     = lam^TB S + (diag(w_upd) K_b)^T V_b   (Step 4, fp32 accumulators, never leaves chip)
//
// with the decay weights of the token recurrence S_t = lam S_{t-1} + k_t v_t^T:
//   forward: mask lam^(i-j) for j <= i, w_inter = lam^(i+1),  w_upd = lam^(TB-1-j)
//   reverse: mask lam^(j-i) for j >= i, w_inter = lam^(TB-i), w_upd = lam^j
// The reverse direction is the same scan run from the last tile to the first; the
// backward pass uses it for dK and dV.  All products are v_mfma_f32_32x32x16_bf16.
//
// LDS layout (bf16, every row split in 16-byte chunks XOR-swizzled by row index):
//   sQ  [TB][D]   natural Q tile          (A^T B operand, Q S A operand)
//   sK  [TB][D]   natural K tile          (A^T A operand)
//   sKT [D][TB]   weighted K^T            (state update A operand)
//   sVT [DV][TB]  V^T                     (P V B operand, state update B operand)
//   sST [DV][D]   S^T rounded to bf16     (Q S B operand)
// In sKT and sVT the positions of each group of 16 are stored in the order
// 0-3, 8-11, 4-7, 12-15, which is the order in which one lane of a 32x32 MFMA
// accumulator holds the rows of P, so P can be fed to the next MFMA directly.
#include "la2_internal.h"

namespace la2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Offset (in bf16 elements) of 16-byte chunk `chunk` of row `row` in a [rows][RL] LDS matrix.
template <int RL>
__device__ __forceinline__ int lds_off(int row, int chunk) {
    constexpr int NCH = RL / 8;
    return row * RL + ((chunk ^ (row & (NCH - 1))) << 3);
}

// Same for the transposed tiles (rows are d or d_v indices, chunks hold 8 positions).  Staging
// writes one column of 8x8 blocks per lane, so a group of lanes hits rows 8 apart; the swizzle
// folds row bits 3.. into the chunk index so those writes and the MFMA fragment reads (32
// consecutive rows) both land on distinct banks.
template <int RL>
__device__ __forceinline__ int lds_off_t(int row, int chunk) {
    constexpr int NCH = RL / 8;
    return row * RL + ((chunk ^ ((row ^ (row >> 3)) & (NCH - 1))) << 3);
}

__device__ __forceinline__ bf16x8 lds_read(const u16 *s, int off) {
    return *reinterpret_cast<const bf16x8 *>(s + off);
}

__device__ __forceinline__ void lds_write(u16 *s, int off, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(s + off) = v;
}

__device__ __forceinline__ u32x4 gload(const u16 *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float bf16_to_f32(unsigned int bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ unsigned int f32_to_bf16(float f) {
    return (unsigned int)__builtin_bit_cast(u16, (__bf16)f);
}

__device__ __forceinline__ unsigned int elem(const u32x4 &x, int e) {
    return (x[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}

// Row (within the tile) of element i of 8-row group rg, in the 0-3,8-11,4-7,12-15 order.
__device__ __forceinline__ int group_row(int rg, int i) {
    return 16 * (rg >> 1) + 4 * (rg & 1) + i + (i >= 4 ? 4 : 0);
}

template <int D, int DV, int TB, Mode MODE>
struct Cfg {
    static constexpr bool kOut = MODE == Mode::Output;
    static constexpr int NTB = TB / 32;          // 32-row blocks of the tile
    static constexpr int NDB = DV / 32;          // 32-column blocks of the value slice
    static constexpr int NKB = D / 32;           // 32-row blocks of the state
    static constexpr int WPT = (kWaves / NTB < NDB) ? kWaves / NTB : NDB;   // waves sharing one row block
    static constexpr int ODB = NDB / WPT;        // value blocks of O per wave
    static constexpr int NSB = NKB * NDB;        // 32x32 blocks of the state
    static constexpr int SPW = NSB > kWaves ? NSB / kWaves : 1;   // state blocks per wave
    // global -> register staging: Q in 16-byte chunks, K and V in 8x8 blocks (one per thread)
    static constexpr int QCH = kOut ? TB * D / 8 : 0;
    static constexpr int QPT = (QCH + kThreads - 1) / kThreads;
    static constexpr int KBLK = (TB / 8) * (D / 8);
    static constexpr int VBLK = (TB / 8) * (DV / 8);
    // LDS carve-up (bf16 elements)
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + (kOut ? TB * D : 0);
    static constexpr int oKT = oK + (kOut ? TB * D : 0);
    static constexpr int oVT = oKT + D * TB;
    static constexpr int oST = oVT + DV * TB;
    static constexpr int kLds = oST + (kOut ? DV * D : 0);
    static_assert(NTB == 2 || NTB == 4, "tile of 64 or 128 positions");
    static_assert(ODB * WPT == NDB && NTB * WPT <= kWaves, "output blocks");
    static_assert(SPW * kWaves == NSB || (SPW == 1 && NSB <= kWaves), "state blocks");
    static_assert(KBLK + VBLK <= kThreads, "one staging block per thread");
    static_assert(kLds * 2 <= 160 * 1024, "LDS");
};

// Row block and part (which ODB value blocks) of O owned by a wave.  Waves w and w + 4
// share a SIMD; the mapping gives each SIMD one short and one long causal row block.
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

template <int D, int DV, int TB, Mode MODE>
struct Staged {
    using C = Cfg<D, DV, TB, MODE>;
    u32x4 q[C::QPT > 0 ? C::QPT : 1];
    u32x4 blk[8];     // rows of this thread's 8x8 block of K (tid < KBLK) or V (KBLK <= tid < KBLK + VBLK)
};

template <int D, int DV, int TB, Mode MODE>
__device__ __forceinline__ void stage_load(Staged<D, DV, TB, MODE> &r, const u16 *a, const u16 *b,
                                           const u16 *c, int64_t t0, int64_t T, int DVT, int tid) {
    using C = Cfg<D, DV, TB, MODE>;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if constexpr (C::kOut) {
#pragma unroll
        for (int s = 0; s < C::QPT; ++s) {
            const int cid = tid + s * kThreads;
            const int row = cid / (D / 8), ch = cid % (D / 8);
            const int64_t t = t0 + row;
            r.q[s] = (cid < C::QCH && t < T) ? gload(a + t * D + ch * 8) : zero;
        }
    }
    if (tid < C::KBLK) {
        const int rg = tid / (D / 8), cc = tid % (D / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t t = t0 + group_row(rg, i);
            r.blk[i] = t < T ? gload(b + t * D + cc * 8) : zero;
        }
    } else if (tid < C::KBLK + C::VBLK) {
        const int bid = tid - C::KBLK;
        const int rg = bid / (DV / 8), cc = bid % (DV / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t t = t0 + group_row(rg, i);
            r.blk[i] = t < T ? gload(c + t * DVT + cc * 8) : zero;
        }
    }
}

// Transpose an 8x8 block of bf16 (rows in x[0..7]) and write column e as one 16-byte chunk.
template <int TB>
__device__ __forceinline__ void write_transposed(u16 *sT, const u32x4 (&x)[8], int rg, int cc) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        u32x4 out;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const unsigned int lo = x[2 * m][e >> 1], hi = x[2 * m + 1][e >> 1];
            out[m] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        lds_write(sT, lds_off_t<TB>(cc * 8 + e, rg), out);
    }
}

// Same, with row i of the block scaled by wrow[i] (rounded once to bf16).
template <int TB>
__device__ __forceinline__ void write_transposed_weighted(u16 *sT, const u32x4 (&x)[8], const float (&wrow)[8],
                                                          int rg, int cc) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        u32x4 out;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const unsigned int lo = f32_to_bf16(bf16_to_f32(elem(x[2 * m], e)) * wrow[2 * m]);
            const unsigned int hi = f32_to_bf16(bf16_to_f32(elem(x[2 * m + 1], e)) * wrow[2 * m + 1]);
            out[m] = lo | (hi << 16);
        }
        lds_write(sT, lds_off_t<TB>(cc * 8 + e, rg), out);
    }
}

template <int D, int DV, int TB, Dir DIR, Mode MODE, bool DECAY>
__device__ __forceinline__ void stage_store(const Staged<D, DV, TB, MODE> &r, u16 *smem, int tid, float l2) {
    using C = Cfg<D, DV, TB, MODE>;
    if constexpr (C::kOut) {
#pragma unroll
        for (int s = 0; s < C::QPT; ++s) {
            const int cid = tid + s * kThreads;
            if (cid < C::QCH) lds_write(smem + C::oQ, lds_off<D>(cid / (D / 8), cid % (D / 8)), r.q[s]);
        }
    }
    if (tid < C::KBLK) {
        const int rg = tid / (D / 8), cc = tid % (D / 8);
        if constexpr (C::kOut) {
#pragma unroll
            for (int i = 0; i < 8; ++i) lds_write(smem + C::oK, lds_off<D>(group_row(rg, i), cc), r.blk[i]);
        }
        if constexpr (DECAY) {
            float wrow[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = group_row(rg, i);
                wrow[i] = __builtin_amdgcn_exp2f((float)(DIR == Dir::Forward ? TB - 1 - j : j) * l2);
            }
            write_transposed_weighted<TB>(smem + C::oKT, r.blk, wrow, rg, cc);
        } else {
            write_transposed<TB>(smem + C::oKT, r.blk, rg, cc);
        }
    } else if (tid < C::KBLK + C::VBLK) {
        const int bid = tid - C::KBLK;
        write_transposed<TB>(smem + C::oVT, r.blk, bid / (DV / 8), bid % (DV / 8));
    }
}

// 4x4 transpose inside each quad of lanes: on entry lane m of the quad holds x[i] = M[i][m];
// on exit it holds x[i] = M[m][i].  Two DPP exchanges (lane xor 1, lane xor 2).
__device__ __forceinline__ float dpp_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ void quad_transpose(float &x0, float &x1, float &x2, float &x3, int lane) {
    const bool b0 = lane & 1, b1 = lane & 2;
    float r = dpp_xor1(b0 ? x0 : x1);
    if (b0) x0 = r; else x1 = r;
    r = dpp_xor1(b0 ? x2 : x3);
    if (b0) x2 = r; else x3 = r;
    r = dpp_xor2(b1 ? x0 : x2);
    if (b1) x0 = r; else x2 = r;
    r = dpp_xor2(b1 ? x1 : x3);
    if (b1) x1 = r; else x3 = r;
}

template <int D, int DV, int TB, Dir DIR, Mode MODE, bool DECAY>
__global__ __launch_bounds__(kThreads, 1) void scan_bf16_kernel(ScanArgs p) {
    using C = Cfg<D, DV, TB, MODE>;
    __shared__ __attribute__((aligned(16))) u16 smem[C::kLds];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, col = lane & 31;

    // work item
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

    const u16 *ga = static_cast<const u16 *>(p.a) + (int64_t)chain * T * D;
    const u16 *gb = static_cast<const u16 *>(p.b) + (int64_t)chain * T * D;
    const u16 *gc = static_cast<const u16 *>(p.c) + (int64_t)chain * T * p.DVT + dv0;
    u16 *gy = C::kOut ? static_cast<u16 *>(p.y) + (int64_t)chain * T * p.DVT + dv0 : nullptr;
    float *gs = p.states ? p.states + ((int64_t)chain * p.nseg + seg) * D * p.DVT + dv0 : nullptr;

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
    const bool init_state = C::kOut && gs != nullptr &&
                            (DIR == Dir::Forward ? seg > 0 : seg < p.nseg - 1);
#pragma unroll
    for (int s = 0; s < C::SPW; ++s) {
        const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            sacc[s][r] = (init_state && s_active) ? gs[(int64_t)d * p.DVT + nb * 32 + col] : 0.0f;
        }
    }

    auto tile_of = [&](int it) -> int64_t { return DIR == Dir::Forward ? tile_lo + it : tile_hi - 1 - it; };

    // S^T (bf16) into LDS for the next tile's right product
    auto write_state_lds = [&]() {
        if constexpr (C::kOut) {
            if (!s_active) return;
#pragma unroll
            for (int s = 0; s < C::SPW; ++s) {
                const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = kb * 32 + 8 * j + 4 * h;
                    u32x2 pk;
                    pk[0] = f32_to_bf16(sacc[s][4 * j + 0]) | (f32_to_bf16(sacc[s][4 * j + 1]) << 16);
                    pk[1] = f32_to_bf16(sacc[s][4 * j + 2]) | (f32_to_bf16(sacc[s][4 * j + 3]) << 16);
                    *reinterpret_cast<u32x2 *>(smem + C::oST + lds_off<D>(nb * 32 + col, d >> 3) + (d & 7)) = pk;
                }
            }
        }
    };

    Staged<D, DV, TB, MODE> st;
    stage_load<D, DV, TB, MODE>(st, ga, gb, gc, tile_of(0) * TB, T, p.DVT, tid);
    stage_store<D, DV, TB, DIR, MODE, DECAY>(st, smem, tid, l2);
    if (ntiles > 1) stage_load<D, DV, TB, MODE>(st, ga, gb, gc, tile_of(1) * TB, T, p.DVT, tid);
    if (init_state) write_state_lds();
    __syncthreads();

    bool state_nonzero = init_state;
    for (int it = 0; it < ntiles; ++it) {
        const int64_t t0 = tile_of(it) * TB;
        const bool update = (MODE == Mode::StateOnly) || (it + 1 < ntiles);

        if constexpr (C::kOut) {
            if (o_active) {
                const u16 *sQ = smem + C::oQ, *sK = smem + C::oK, *sVT = smem + C::oVT, *sST = smem + C::oST;
                const int qrow = tb * 32 + col;

                f32x16 oacc[C::ODB];
#pragma unroll
                for (int n = 0; n < C::ODB; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0f;

                // Step 3: inter-tile right product, rows weighted by w_inter
                if (state_nonzero) {
#pragma unroll 2
                    for (int ks = 0; ks < D / 16; ++ks) {
                        const bf16x8 qf = lds_read(sQ, lds_off<D>(qrow, 2 * ks + h));
#pragma unroll
                        for (int n = 0; n < C::ODB; ++n)
                            oacc[n] = mfma(qf, lds_read(sST, lds_off<D>((db0 + n) * 32 + col, 2 * ks + h)), oacc[n]);
                    }
                    if constexpr (DECAY) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int i = tb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                            const float w = pw(DIR == Dir::Forward ? i + 1 : TB - i);
#pragma unroll
                            for (int n = 0; n < C::ODB; ++n) oacc[n][r] *= w;
                        }
                    }
                }

                // Step 2: intra-tile masked left product, one 32x32 block of A^T at a time
                const int ulo = DIR == Dir::Forward ? 0 : tb;
                const int uhi = DIR == Dir::Forward ? tb : C::NTB - 1;
                const int tcol = tb * 32 + col;
                for (int u = ulo; u <= uhi; ++u) {
                    f32x16 acc;
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll 4
                    for (int ks = 0; ks < D / 16; ++ks)
                        acc = mfma(lds_read(sK, lds_off<D>(u * 32 + col, 2 * ks + h)),
                                   lds_read(sQ, lds_off<D>(qrow, 2 * ks + h)), acc);
                    // causal decay mask: only the diagonal block has masked entries
                    bf16x8 pf[2];
                    if (u == tb) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int tp = u * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                            const int diff = DIR == Dir::Forward ? tcol - tp : tp - tcol;
                            const float v = diff >= 0 ? (DECAY ? acc[r] * pw(diff) : acc[r]) : 0.0f;
                            pf[r >> 3][r & 7] = (__bf16)v;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int tp = u * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                            const int diff = DIR == Dir::Forward ? tcol - tp : tp - tcol;
                            pf[r >> 3][r & 7] = (__bf16)(DECAY ? acc[r] * pw(diff) : acc[r]);
                        }
                    }
#pragma unroll
                    for (int x = 0; x < 2; ++x)
#pragma unroll
                        for (int n = 0; n < C::ODB; ++n)
                            oacc[n] = mfma(pf[x],
                                           lds_read(sVT, lds_off_t<TB>((db0 + n) * 32 + col, 4 * u + 2 * x + h)),
                                           oacc[n]);
                }

                // store O: a quad transpose gives each lane 4 consecutive columns of one row
#pragma unroll
                for (int n = 0; n < C::ODB; ++n) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float x0 = oacc[n][4 * j], x1 = oacc[n][4 * j + 1], x2 = oacc[n][4 * j + 2],
                              x3 = oacc[n][4 * j + 3];
                        quad_transpose(x0, x1, x2, x3, lane);
                        const int64_t t = t0 + tb * 32 + 8 * j + 4 * h + (lane & 3);
                        if (t < T) {
                            u32x2 pk;
                            pk[0] = f32_to_bf16(x0) | (f32_to_bf16(x1) << 16);
                            pk[1] = f32_to_bf16(x2) | (f32_to_bf16(x3) << 16);
                            *reinterpret_cast<u32x2 *>(gy + t * p.DVT + (db0 + n) * 32 + (col & ~3)) = pk;
                        }
                    }
                }
            }
        }

        // Step 4: state update S = lam^TB S + (w_upd K)^T V, fp32 accumulators
        if (update) {
            if (s_active) {
                if constexpr (DECAY) {
                    const float f = pw(TB);
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) sacc[s] *= f;
                }
                const u16 *sKT = smem + C::oKT, *sVT = smem + C::oVT;
#pragma unroll 2
                for (int x = 0; x < TB / 16; ++x) {
#pragma unroll
                    for (int s = 0; s < C::SPW; ++s) {
                        const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
                        sacc[s] = mfma(lds_read(sKT, lds_off_t<TB>(kb * 32 + col, 2 * x + h)),
                                       lds_read(sVT, lds_off_t<TB>(nb * 32 + col, 2 * x + h)), sacc[s]);
                    }
                }
            }
            state_nonzero = true;
        }

        __syncthreads();                       // every wave is done with this tile's LDS
        if (update) write_state_lds();
        if (it + 1 < ntiles) {
            stage_store<D, DV, TB, DIR, MODE, DECAY>(st, smem, tid, l2);
            if (it + 2 < ntiles) stage_load<D, DV, TB, MODE>(st, ga, gb, gc, tile_of(it + 2) * TB, T, p.DVT, tid);
        }
        __syncthreads();
    }

    if constexpr (MODE == Mode::StateOnly) {
        if (s_active) {
#pragma unroll
            for (int s = 0; s < C::SPW; ++s) {
                const int sb = wave * C::SPW + s, kb = sb / C::NDB, nb = sb % C::NDB;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    gs[(int64_t)d * p.DVT + nb * 32 + col] = sacc[s][r];
                }
            }
        }
    }
}

template <int D, int DV, int TB, Dir DIR, Mode MODE>
hipError_t launch_one(const ScanArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)a.chains * a.seg_count * a.nslice;
    if (a.decay)
        hipLaunchKernelGGL((scan_bf16_kernel<D, DV, TB, DIR, MODE, true>), dim3((unsigned)items), dim3(kThreads), 0,
                           s, a);
    else
        hipLaunchKernelGGL((scan_bf16_kernel<D, DV, TB, DIR, MODE, false>), dim3((unsigned)items), dim3(kThreads),
                           0, s, a);
    return hipGetLastError();
}

template <int D, int DV, int TB>
hipError_t launch_dm(const ScanArgs &a, Dir dir, Mode mode, hipStream_t s) {
    if (dir == Dir::Forward)
        return mode == Mode::Output ? launch_one<D, DV, TB, Dir::Forward, Mode::Output>(a, s)
                                    : launch_one<D, DV, TB, Dir::Forward, Mode::StateOnly>(a, s);
    return mode == Mode::Output ? launch_one<D, DV, TB, Dir::Reverse, Mode::Output>(a, s)
                                : launch_one<D, DV, TB, Dir::Reverse, Mode::StateOnly>(a, s);
}

template <int D, int DV>
hipError_t launch_tb(const ScanArgs &a, int TB, Dir dir, Mode mode, hipStream_t s) {
    return TB == 64 ? launch_dm<D, DV, 64>(a, dir, mode, s) : launch_dm<D, DV, 128>(a, dir, mode, s);
}

}  // namespace

bool bf16_supported(int D, int DV, int TB) {
    return (D == 64 || D == 128) && (DV == 64 || DV == 128) && (TB == 64 || TB == 128);
}

hipError_t launch_scan_bf16(const ScanArgs &a, int D, int DV, int TB, Dir dir, Mode mode, hipStream_t s) {
    if (!bf16_supported(D, DV, TB)) return hipErrorInvalidValue;
    if (D == 64) return DV == 64 ? launch_tb<64, 64>(a, TB, dir, mode, s) : launch_tb<64, 128>(a, TB, dir, mode, s);
    return DV == 64 ? launch_tb<128, 64>(a, TB, dir, mode, s) : launch_tb<128, 128>(a, TB, dir, mode, s);
}

}  // namespace la2
