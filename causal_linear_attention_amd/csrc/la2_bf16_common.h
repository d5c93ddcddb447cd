// la2_bf16_common.h -- device helpers shared by the bf16 MFMA kernels (gfx950).
//
// Tiles live in LDS in natural row-major layout with 16-byte chunks XOR-swizzled by row; MFMA
// operand fragments come from plain 16-byte reads or from ds_read_b64_tr_b16 transpose reads; HBM
// is accessed through buffer resources whose range check zero-fills loads and drops stores past
// the end of a sequence.
#pragma once

#include "la2_internal.h"

namespace la2 {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Element offset of 16-byte chunk `chunk` of row `row` in a row-major [rows][RL] bf16 LDS tile.
// RL = 128: chunk ^ (row ^ 4 (row & 3)) mod 16 spreads both 32 consecutive rows at one chunk
// (fragment reads) and rows {r..r+3, r+8..r+11} at four chunks (transpose reads) over all banks.
template <int RL>
__device__ __forceinline__ int swz(int row) {
    if constexpr (RL == 128)
        return (row ^ ((row & 3) << 2)) & 15;
    else
        return (row >> 1) & 7;
}

template <int RL>
__device__ __forceinline__ int nat_off(int row, int chunk) {
    return row * RL + ((chunk ^ swz<RL>(row)) << 3);
}

__device__ __forceinline__ bf16x8 lds_read(const u16 *s, int off) {
    return *reinterpret_cast<const bf16x8 *>(s + off);
}

__device__ __forceinline__ void lds_write(u16 *s, int off, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(s + off) = v;
}

__device__ __forceinline__ s16x4 tr_read(const u16 *s, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(s + off));
}

// MFMA operand fragment (either side) from a natural [positions][RL] tile: lane l gets column
// n0 + l % 32 and 8 positions.  PERM = false: positions k0 + 8h + 0..7 (h = l / 32), the order
// of a plain 16-byte read; PERM = true: k0 + {4h..4h+3, 8+4h..8+4h+3}, the order in which an
// MFMA accumulator lane holds the rows of P.
template <int RL, bool PERM>
__device__ __forceinline__ bf16x8 frag_tr(const u16 *s, int k0, int n0, int lane) {
    const int g = lane >> 4, j = lane & 15, h = g >> 1;
    const int col = n0 + 16 * (g & 1) + 4 * (j & 3);
    const int r0 = k0 + (PERM ? 4 * h : 8 * h) + (j >> 2);
    const int r1 = r0 + (PERM ? 8 : 4);
    // assemble from whole dwords: per-element 16-bit extraction of the builtin's result is
    // mis-lowered by this compiler (every element comes out as element 0)
    const u32x2 a = __builtin_bit_cast(u32x2, tr_read(s, nat_off<RL>(r0, col >> 3) + (col & 7)));
    const u32x2 b = __builtin_bit_cast(u32x2, tr_read(s, nat_off<RL>(r1, col >> 3) + (col & 7)));
    const u32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// Cache policy of the tile streams: every tile is read (or written) once per launch, so the loads
// and stores carry the nontemporal hint (nt, bit 1 of the cache-policy operand), which keeps
// them from displacing reusable lines in L2 and the memory-side cache.
constexpr int kStreamCpol = 2;

// Buffer resource over `bytes` bytes from `base`: loads past the end return 0 and stores past
// the end are dropped by the hardware range check, which is what handles a ragged last tile.
// Every caller addresses at most one tile past `base`, so a range longer than 1 GiB is cut to
// 1 GiB: the 32-bit record count must not wrap on chains of more than 2^31 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    constexpr int64_t kCap = (int64_t)1 << 30;
    const int n = bytes <= 0 ? 0 : (int)(bytes < kCap ? bytes : kCap);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kStreamCpol));
}

__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, int byte_off, const u32x4 &v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                           byte_off, 0, kStreamCpol);
}

__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, int byte_off, const u32x2 &v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r,
                                          byte_off, 0, kStreamCpol);
}

__device__ __forceinline__ unsigned int f32_to_bf16(float f) {
    return (unsigned int)__builtin_bit_cast(u16, (__bf16)f);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed pair of bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ unsigned int pack_bf16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2));
}

// Direct global -> LDS loads of the RL-wide rows [0, NR) of a tile (no registers involved).  Each
// 16-byte lane load lands at the next 16 bytes of LDS, so lane l of load i fills LDS chunk
// 64 i + l and fetches the global chunk that the XOR swizzle assigns there.  Rows past the
// descriptor's range arrive as zeros.  Completion is tracked by this wave's vmcnt.
template <int RL, int NR>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, u16 *dst, int gstride, int wave, int lane) {
    constexpr int CPR = RL / 8, NL = NR * CPR / 64;
    static_assert(NL % kWaves == 0, "whole loads per wave");
#pragma unroll
    for (int s = 0; s < NL / kWaves; ++s) {
        const int i = wave + kWaves * s, c = 64 * i + lane, row = c / CPR, lc = (c % CPR) ^ swz<RL>(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 512 * i), 16,
                                                 (row * gstride + lc * 8) * 2, 0, 0, kStreamCpol);
    }
}

// Lanes l and l + 32 (h = l / 32) hold the two 8-byte halves (h = 0 the first) of the 16-byte
// chunks `a` and `b`.  Returns chunk `a` whole in lanes 0..31 and chunk `b` whole in lanes 32..63.
// v_permlane32_swap(x, y) leaves, in lane l < 32, (x of lane l, x of lane l + 32) and, in lane
// l >= 32, (y of lane l - 32, y of lane l): one swap per dword pairs up the halves.
__device__ __forceinline__ u32x4 join_halves(const u32x2 &a, const u32x2 &b) {
    const auto r0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
    const u32x4 w = {r0[0], r1[0], r0[1], r1[1]};
    return w;
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS hand-over only: waits for this wave's LDS operations, not for its
// global loads, so the next tile's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Decay: the state update's copy of a [TB][D] key-role tile, row j scaled by w_upd(j) (lam^(TB-1-j)
// forward, lam^j reverse) and rounded once to bf16 (same swizzled layout, so a chunk keeps its offset).
// `extra` adds lam^extra to every row (a tile's own decay factor when the tiles are not visited in
// scan order).
template <int D, int TB, Dir DIR>
__device__ __forceinline__ void build_kw(const u16 *sk, u16 *skw, int tid, float l2, int extra = 0) {
#pragma unroll
    for (int s = 0; s < TB * D / 8 / kThreads; ++s) {
        const int c = tid + kThreads * s, row = c / (D / 8);
        const float w = __builtin_amdgcn_exp2f((float)((DIR == Dir::Forward ? TB - 1 - row : row) + extra) * l2);
        u32x4 x = *reinterpret_cast<const u32x4 *>(sk + 8 * c);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            x[m] = f32_to_bf16(__uint_as_float(x[m] << 16) * w) | (f32_to_bf16(__uint_as_float(x[m] & 0xffff0000u) * w) << 16);
        *reinterpret_cast<u32x4 *>(skw + 8 * c) = x;
    }
}

}  // namespace dev
}  // namespace la2
