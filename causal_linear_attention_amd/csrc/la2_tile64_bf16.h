// la2_tile64_bf16.h -- pieces shared by the bf16 kernels that walk 64-position tiles at d = d_v = 128
// with one output unit of 32 rows x 64 columns per wave (la2_bwd1_bf16.hip, la2_fwd1_bf16.hip):
// per-lane LDS offsets, fragment reads, the causal score block and the unit's products.
//
// Tiles are [rows][128] bf16 in LDS with 16-byte chunks XOR-swizzled by row (nat_off); MFMA
// accumulators hold O^T (lane col = output row), as in la2_bf16_common.h.
#pragma once

#include "la2_bf16_common.h"

namespace la2 {
namespace t64 {

using namespace dev;

constexpr int D1 = 128;              // d = d_v
constexpr int TB1 = 64;              // positions per tile
constexpr int kTile1 = TB1 * D1;     // bf16 elements of one input tile
constexpr int KS1 = D1 / 16;         // contraction steps over d

// Per-lane LDS offsets (bf16 elements), computed once so that every LDS access in the tile loop is a
// per-lane register plus a compile-time or per-block offset.  Tiles are [rows][128] with 16-byte
// chunks XOR-swizzled by row (nat_off); the swizzle depends only on row % 16, so within a lane it is
// the same for every row block, and the chunk index splits into bits the block offset cannot carry.
struct LaneOff {
    int pl[8];          // row col, chunk 2m + h (plain fragment reads; + 128 row0)
    int trn[4][2];      // transposed reads without permutation at k0 = 0 of column block nb (+ 128 k0),
                        // first and second 8-byte piece
    int trc[2][2][2];   // [PERM][n][piece] the same for this wave's column blocks 2ch + n
    int pw[2][4];       // row col, chunk 4(2ch + i) + g, 8-byte half h: where accumulator entries
                        // 4g..4g+3 of this wave's state blocks with rows kb = 2ch + i land in a
                        // transposed state
    int po[2][4];       // the same in a 64-column output staging row (chunk 4n + g)
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
        for (int g = 0; g < 4; ++g) {
            L.pw[i][g] = nat_off<D1>(col, 4 * (2 * ch + i) + g) + 4 * h;
            L.po[i][g] = col * 64 + (((4 * i + g) ^ ((col >> 1) & 7)) << 3) + 4 * h;
        }
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

// bf16x8 with every sign bit xor-ed with `sign` (0x80008000: every element negated, exactly; 0: as is).
__device__ __forceinline__ bf16x8 flip8(const bf16x8 &f, unsigned int sign) {
    u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int m = 0; m < 4; ++m) u[m] ^= sign;
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void lds_write8(u16 *s, int off, const u32x2 &v) {
    *reinterpret_cast<u32x2 *>(s + off) = v;
}

// P of one 32 x 32 score block as the B operand of the value products.  Accumulator r of lane
// (h, col) holds source row 8(r/4) + 4h + r%4 against output row col; pairs (2p, 2p + 1) are rounded
// to bf16 together.  In the diagonal block the entries on the wrong side of the causal mask are
// zeroed first (SRC_BEFORE: sources at or before the output row are kept, else at or after).  RS:
// the lane's kept fp32 scores are also added to *rs (half of the output row's sum over the block).
// DEC (a decay): each score is multiplied by wt[r] first (decay_weights below).  ADD: ad[r] is added
// to each score first (a value per source row: the normalized form's denominator gradient).
template <bool SRC_BEFORE, bool DIAG, bool RS = false, bool DEC = false, bool ADD = false>
__device__ __forceinline__ void block_p(const f32x16 &acc, bf16x8 (&pf)[2], int h, int col, float *rs,
                                        const float (&wt)[16], const float (&ad)[16]) {
    u32x4 w[2];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        float a = acc[2 * p], b = acc[2 * p + 1];
        if constexpr (DEC) {
            a *= wt[2 * p];
            b *= wt[2 * p + 1];
        }
        if constexpr (ADD) {
            a += ad[2 * p];
            b += ad[2 * p + 1];
        }
        if (DIAG) {
            const int dist = 4 * h - col + 8 * (p >> 1) + 2 * (p & 1);   // source - output of entry 2p
            a = (SRC_BEFORE ? dist <= 0 : dist >= 0) ? a : 0.0f;
            b = (SRC_BEFORE ? dist + 1 <= 0 : dist + 1 >= 0) ? b : 0.0f;
        }
        if constexpr (RS) *rs += a + b;
        w[p >> 2][p & 3] = pack_bf16(a, b);
    }
    pf[0] = __builtin_bit_cast(bf16x8, w[0]);
    pf[1] = __builtin_bit_cast(bf16x8, w[1]);
}

// The intra-tile contribution of source block u to a unit: scores of the block's 32 source rows
// against the unit's 32 output rows (B operand bf), then P times the value rows of the block.  ADD:
// sAdd[j] (fp32, per source position j of the tile) is added to every score of source row j.
template <bool SRC_BEFORE, bool DIAG, bool RS, bool DEC, bool ADD = false>
__device__ __forceinline__ void intra_block(f32x16 (&oacc)[2], const bf16x8 (&bf)[KS1], const u16 *sA,
                                            const u16 *sC, int u, const LaneOff &L, int h, int col, float *rs,
                                            const float (&wt)[16], const float *sAdd = nullptr) {
    const f32x16 zero = {};
    f32x16 acc = mfma(rd_plain(sA, u * 32, 0, L), bf[0], zero);
#pragma unroll
    for (int ks = 1; ks < KS1; ++ks) acc = mfma(rd_plain(sA, u * 32, ks, L), bf[ks], acc);
    float add[16] = {};
    if constexpr (ADD) {
        // accumulator entries 4g..4g+3 are source rows u*32 + 8g + 4h .. + 3: one 16-byte read each
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 v = *reinterpret_cast<const float4 *>(sAdd + u * 32 + 8 * g + 4 * h);
            add[4 * g] = v.x;
            add[4 * g + 1] = v.y;
            add[4 * g + 2] = v.z;
            add[4 * g + 3] = v.w;
        }
    }
    bf16x8 pf[2];
    block_p<SRC_BEFORE, DIAG, RS, DEC, ADD>(acc, pf, h, col, rs, wt, add);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int n = 0; n < 2; ++n) oacc[n] = mfma(rd_tr(sC, u * 32 + 16 * x, L.trc[1][n]), pf[x], oacc[n]);
}

// The weights of a decay lam = 2^l2, per lane (h, col) of a unit in row block orow, for accumulator
// entry r (output row t = col, source row s = 8(r/4) + 4h + r%4 within their blocks).  Forward
// (SRC_BEFORE): wd[r] = lam^(t - s) in the diagonal score block where s <= t, else 0; wf[r] =
// lam^(32 + t - s) in the full block before it (row block 1 only); wi = lam^(orow*32 + col + 1), the
// inter product's weight (the state is the one before the tile).  Reverse: wd[r] = lam^(s - t) where
// s >= t, else 0; wf[r] = lam^(32 + s - t) in the full block after it (row block 0 only); wi =
// lam^(64 - orow*32 - col) (the state is the one after the tile).  Every exponent is non-negative.
struct DecayW {
    float wd[16], wf[16], wi;
};

template <bool SRC_BEFORE>
__device__ __forceinline__ DecayW decay_weights(float l2, int orow, int lane) {
    const int h = lane >> 5, col = lane & 31;
    DecayW w;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int s = 8 * (r >> 2) + 4 * h + (r & 3), dist = SRC_BEFORE ? col - s : s - col;
        w.wd[r] = dist >= 0 ? exp2f(l2 * (float)dist) : 0.0f;
        w.wf[r] = orow == (SRC_BEFORE ? 1 : 0) ? exp2f(l2 * (float)(32 + dist)) : 0.0f;
    }
    w.wi = exp2f(l2 * (float)(SRC_BEFORE ? orow * 32 + col + 1 : TB1 - orow * 32 - col));
    return w;
}

// One output unit of a wave: columns 64ch..64ch+63 (two 32-column blocks) of the output rows in block
// `orow`, as O^T accumulators (lane col holds output row orow*32 + col): the inter product of the
// state copy sSt (INTER_PLAIN: its rows are the output columns, read plain; else its columns, read
// transposed) with the unit's output-row tile sB, then the intra-tile scores of the source-row tile
// sA against sB over the causal source blocks (SRC_BEFORE: sources at or before the output row,
// else at or after) times the value tile sC.  The inter product always runs (a state that is still
// zero contributes zeros), so the first contraction step starts from a zero accumulator operand
// instead of cleared registers.
// DEN (the normalized form): *den = the lane's half of the output row's denominator: its half of the
// row's kept fp32 scores, plus (lanes 0..31) the product of the sB row with a vector z (the prefix sum
// of the source rows before the tile) that sZ holds as a [32][128] tile whose row 0 is z rounded to
// bf16, row 1 the rounding's remainder rounded to bf16, and the other rows zero; the partner lane
// (lane ^ 32) holds the other half of the scores.
// DEC (a decay): the inter product is weighted by dw.wi and the scores by dw.wd, wf (decay_weights).
// ADD: sAdd[j] (fp32, per source position j of the tile) is added to every score of source row j
// before it is masked and packed.
template <bool SRC_BEFORE, bool INTER_PLAIN, bool DEN = false, bool DEC = false, bool ADD = false>
__device__ __forceinline__ void unit_products(f32x16 (&oacc)[2], const u16 *sB, const u16 *sA, const u16 *sC,
                                              const u16 *sSt, int orow, int ch, int lane, const LaneOff &L,
                                              float *den, const u16 *sZ, const DecayW &dw,
                                              const float *sAdd = nullptr) {
    const int h = lane >> 5, col = lane & 31;
    bf16x8 bf[KS1];
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) bf[ks] = rd_plain(sB, orow * 32, ks, L);
    float dd = 0.0f;
    if constexpr (DEN) {
        // rows 0 and 1 of the product land in accumulator entries 0 and 1 of lanes 0..31 (h = 0); the
        // entries of lanes 32..63 are rows 4 and 5, zero
        const f32x16 zero = {};
        f32x16 dacc = mfma(rd_plain(sZ, 0, 0, L), bf[0], zero);
#pragma unroll
        for (int ks = 1; ks < KS1; ++ks) dacc = mfma(rd_plain(sZ, 0, ks, L), bf[ks], dacc);
        dd = dacc[0] + dacc[1];
    }
    // fully unrolled: bf[] must be indexed by constants (a runtime index into a register array is
    // lowered to chains of selects)
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const bf16x8 a = INTER_PLAIN ? rd_plain(sSt, (2 * ch + n) * 32, ks, L) : rd_tr(sSt, 16 * ks, L.trc[0][n]);
            oacc[n] = mfma(a, bf[ks], ks == 0 ? zero : oacc[n]);
        }
    if constexpr (DEC) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[n][e] *= dw.wi;
    }
    // intra-tile: the whole source block before (SRC_BEFORE) or after the diagonal, where there is one,
    // then the diagonal block
    if (SRC_BEFORE ? orow == 1 : orow == 0)
        intra_block<SRC_BEFORE, false, DEN, DEC, ADD>(oacc, bf, sA, sC, SRC_BEFORE ? 0 : 1, L, h, col, &dd, dw.wf,
                                                      sAdd);
    intra_block<SRC_BEFORE, true, DEN, DEC, ADD>(oacc, bf, sA, sC, orow, L, h, col, &dd, dw.wd, sAdd);
    if constexpr (DEN) *den = dd;
}

// The unit without a denominator or a decay.
template <bool SRC_BEFORE, bool INTER_PLAIN>
__device__ __forceinline__ void unit_products(f32x16 (&oacc)[2], const u16 *sB, const u16 *sA, const u16 *sC,
                                              const u16 *sSt, int orow, int ch, int lane, const LaneOff &L) {
    const DecayW none = {};   // not read
    unit_products<SRC_BEFORE, INTER_PLAIN, false, false>(oacc, sB, sA, sC, sSt, orow, ch, lane, L, nullptr, nullptr,
                                                         none);
}

}  // namespace t64
}  // namespace la2
