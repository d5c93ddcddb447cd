// la2_internal.h -- declarations shared by the library's own translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace la2 {

// One launch of the tile-scan kernel over a set of (chain, segment, value-slice)
// work items.  Roles follow the attention output y_t = sum_s w(t, s) (a_t . b_s) c_s:
//   a = "query" [chains, T, D], b = "key" [chains, T, D], c = "value" [chains, T, DVT].
// Forward: (q, k, v) -> o.  Backward: dq = scan(do, v, k); dk = reverse scan(v, do, q);
// dv = reverse scan(k, q, do)  (the three are fused where a kernel supports it).
struct ScanArgs {
    const void *a;
    const void *b;
    const void *c;
    void *y;               // output [chains, T, DVT] (unused in state-only launches)
    const float *decay;    // [H] or nullptr (lam = 1)
    float *states;         // fp32 [chains, nsub, D, DVT]: segment start states / segment deltas
    int states_t;          // 1: output launches read the start states transposed, [chains, nsub, DVT, D]
    int has_init;          // output launches: the first segment in scan order also starts from `states`
                           // (forward: a carried-in state; reverse: the gradient of a carried-out
                           // state, attached at the chain's last position)
    float *state_out;      // output launches: fp32 [chains, D, DVT], forward: the final state; reverse:
                           // lam times the state at position 0 (gradient of a carried-in state)
    int64_t T;
    int H;
    int DVT;               // full value width (row stride of c and y)
    int nseg;              // segments per chain
    int seg_tiles;         // tiles per segment
    int seg_first;         // first segment index handled by this launch
    int seg_count;         // segments per chain handled by this launch
    int nslice;            // value slices per chain (DVT / slice width)
    int chains;            // B * H
    // `states` holds nsub entries per chain, `sub` per segment of this launch (state-only launches
    // may run finer segments than the output launch that reads them); output segment s starts from
    // entry state_index(s)
    int sub;
    int nsub;
    const float *den;      // forward output launches: fp32 [chains, T], y_t is divided by den_t before it
                           // is stored (the normalized form), or nullptr
};

// Entry of the states array a segment starts from: its first sub-segment in the forward direction,
// its last one in the reverse direction.
__host__ __device__ inline int state_index(int seg, int sub, int nsub, bool reverse) {
    if (!reverse) return seg * sub;
    const int i = seg * sub + sub - 1;
    return i < nsub - 1 ? i : nsub - 1;
}

// Kernel families.
enum class Dir { Forward, Reverse };
enum class Mode { Output, StateOnly };

// Launchers (return hipGetLastError() after the launch).
// Output pass of the bf16 tile scan (state-only passes: launch_state_bf16).
hipError_t launch_scan_bf16(const ScanArgs &a, int D, int DV, int TB, Dir dir, hipStream_t s);
hipError_t launch_scan_f32(const ScanArgs &a, int D, int DV, int TB, Dir dir, Mode mode,
                           hipStream_t s);
// State-only pass of bf16 split chains (its own 64-position tiles, several in flight); `a` gives
// the segments in tiles of TB positions, TB a multiple of 64.
hipError_t launch_state_bf16(const ScanArgs &a, int D, int DV, int TB, Dir dir, hipStream_t s);
// Turns per-segment deltas into per-segment start states, in place; `init` ([chains, elems] or
// nullptr) is the state the first segment in scan order starts from (reverse: the gradient of a
// carried-out state, attached at the chain's last position, which the first step weights with
// lam^init_len, init_len = the last segment's length - 1).
hipError_t launch_segment_prefix(float *states, const float *decay, int chains, int H, int nseg,
                                 int64_t seg_len, int64_t elems, Dir dir, hipStream_t s,
                                 const float *init = nullptr, int64_t init_len = 0);

// One token of the recurrence for every chain: state <- lam state + k v^T (fp32 [chains, D, DV], in
// place), o = state^T q.  q, k: [chains, D]; v, o: [chains, DV]; bf16 (dtype 1) or fp32 (0).
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *decay, void *o, float *state,
                         int chains, int H, int D, int DV, int dtype, hipStream_t s);

// Normalized output (feature map phi: 0 identity, 1 elu + 1) and its backward.  launch_vscan runs
// the decayed d-vector scans of the denominator (modes in la2_norm.hip: 0 forward segment sums of
// phi(k), 1 den_t = phi(q_t) . z_t with phi(q), phi(k) written where pq / pk are given, 2 the
// denominator's part of dq, 3 reverse segment sums of dden_t phi(q_t), 4 the denominator's part of
// dk; the division by den is done by the numerator's output launch, ScanArgs::den),
// launch_grad_rows forms dn = do / den and dden = -(do . o) / den.
struct DenArgs {
    const void *q, *k;     // [chains, T, D], phi applied inside
    void *pq, *pk;         // [chains, T, D] phi(q), phi(k) out (mode 1), or nullptr
    float *den;            // fp32 [chains, T]: out (mode 1)
    const float *dden;     // fp32 [chains, T]: in (modes 2-4)
    void *g;               // [chains, T, D]: dq (mode 2) or dk (mode 4), updated in place
    const float *decay;    // [H] or nullptr (lam = 1)
    float *zseg;           // fp32 [chains, nseg, D]: per-segment sums
    float *msum;           // fp32 [chains, nseg, D]: plain (undecayed) per-segment sums of phi(k) (mode 5 out,
                           // modes 6 and 7 in: the chain's mean m of phi(k))
    void *kap;             // [chains, T, D]: phi(k) - m (mode 6 out)
    const void *u;         // [chains, T, D]: the scan of (dout, v, phi(k) - m) (mode 7 in)
    const float *arow;     // fp32 [chains, T]: dout_t . (decayed prefix sum of v)_t (mode 7 in)
    float *dden_out;       // fp32 [chains, T]: where mode 7 also writes dden_t = -(dout_t . o_t) / den_t, or nullptr
    int64_t T;
    int64_t seg_len;       // positions per segment, a multiple of 64
    int H;
    int nseg;
    int chains;
};
hipError_t launch_vscan(const DenArgs &a, int D, int dtype, int fmap, int mode, hipStream_t s);
hipError_t launch_grad_rows(const void *o, const void *dout, const float *den, void *dn, float *dden, int64_t rows,
                            int DV, int dtype, hipStream_t s);

// The recurrence run token by token (comparison with the tiled scan): o for every chain, state in
// registers from zero.  q, k: [chains, T, D]; v, o: [chains, T, DV]; bf16 (dtype 1) or fp32 (0).
hipError_t launch_serial(const void *q, const void *k, const void *v, const float *decay, void *o, int chains, int H,
                         int64_t T, int D, int DV, int dtype, hipStream_t s);

// Which (D, DV, TB) the kernels are compiled for.
bool bf16_supported(int D, int DV, int TB);
bool f32_supported(int D, int DV, int TB);

// Fused reverse pass of the bf16 backward: dk and dv of each (chain, segment) in one walk over its
// tiles of kDkdvTile positions, from the reverse state R = sum lam^(s-t) q_s do_s^T (d = d_v).
constexpr int kDkdvTile = 64;
struct DkdvArgs {
    const void *q, *k, *v, *dout;
    void *dk, *dv;
    const float *decay;    // [H] or nullptr (lam = 1)
    const float *states;   // fp32 [chains, nsub, D, D] start states of R, or nullptr when not split
    int64_t T;
    int H;
    int nseg;
    int seg_tiles;
    int chains;
    int sub;               // entries of `states` per segment (see ScanArgs)
    int nsub;
    int has_init;          // the last segment also starts from `states`: a gradient of the carried-out
                           // state, attached at the chain's last position
    float *state_out;      // fp32 [chains, D, D]: lam R_0 (gradient of a carried-in state), or nullptr
};
bool dkdv_supported(int D, int DV);
hipError_t launch_dkdv_bf16(const DkdvArgs &a, int D, hipStream_t s);

// The forward-direction output scan without decay at d = d_v = 128, bf16 (la2_fwd1_bf16.hip): y_t =
// sum_{s<=t} (a_t . b_s) c_s + a_t S_in for each (chain, segment) over 64-position tiles, producer
// waves holding S = sum b^T c in registers beside the consumer waves forming y.
struct Fwd1Args {
    const void *q, *k, *v;  // query, key and value roles [chains, T, 128]
    void *y;                // output [chains, T, 128]
    int64_t T;
    int64_t seg_len;        // positions per segment, a multiple of 64
    int nseg;
    int chains;
    const float *states;    // fp32 segment start states ([chains, nsub, D, D]) or nullptr (unsplit)
    int states_t;           // 1: the entries are stored transposed ([DV][D])
    int sub, nsub;          // states entry of segment s: state_index(s, sub, nsub, false)
    float *state_out;       // fp32 [chains, D, D]: the state after the last position, or nullptr
    // the normalized form (norm = 1: identity feature map, 2: elu + 1; 0: the plain scan): each output
    // row is divided by phi(q_t) . z_t, z_t the prefix sum of phi(k_s); unsplit chains only (nseg = 1).
    // norm = 3 (identity), 4 (elu + 1): the plain scan with the value role v replaced by phi(v) - m, m
    // the chain's mean of phi(v) from msum (the normalized backward's centered keys); unsplit only
    int norm;
    void *pq, *pk;          // where phi(q), phi(k) are also written (bf16 [chains, T, 128]), or nullptr
    float *den;             // where the denominators are also written (fp32 [chains, T]), or nullptr;
                            //   norm 3, 4: q_t . (the prefix sum of k through t), the rows undivided
    float *msum;            // where each msum_seg-position segment's sum of phi(k) is also written (fp32
    int64_t msum_seg;       //   [chains, ceil(T / msum_seg), 128]; msum_seg a multiple of 64), or nullptr
    const float *decay;     // per-head decay lam ([H] fp32, chain c is head c % H), or nullptr for lam = 1;
    int H;                  //   the plain scan only
};
hipError_t launch_fwd1_bf16(const Fwd1Args &a, hipStream_t s);

// The whole backward without decay in one reverse walk (la2_bwd1_bf16.hip): dq, dk and dv of each
// (chain, segment) over kBwd1Tile-position tiles, d = d_v = 128, bf16.  The forward state is carried
// backwards from the state after the segment (the next segment's start state, or the chain's final
// state for the last segment), the reverse state forwards from the state at the segment's end.
constexpr int kBwd1Tile = 64;
struct Bwd1Args {
    const void *q, *k, *v, *dout;
    void *dq, *dk, *dv;
    int64_t T;
    int nseg;
    int seg_tiles;         // tiles of kBwd1Tile positions per segment
    int chains;
    const float *s_states; // fp32 [chains, s_nsub, D, D]: forward segment start states (segment p starts
    int s_sub;             //   from entry p * s_sub), or nullptr when not split
    int s_nsub;
    const float *s_final;  // fp32 [chains, D, D]: each chain's state after its last position
    const float *r_states; // fp32 [chains, r_nsub, D, D]: reverse states at the segments' ends, or nullptr
    int r_sub;
    int r_nsub;
    // r_compose != 0: r_states holds the reverse state pass's per-piece deltas instead (no prefix ran),
    // and each segment sums the deltas of the pieces after it, r_piece_len positions each, itself
    int r_compose;
    int64_t r_piece_len;
    // dq = nullptr: dk and dv only (the dK/dV pass of the two-pass backward; s_states, s_final unused),
    // with the per-head decay lam ([H] fp32, chain c is head c % H) or nullptr for lam = 1
    const float *decay;
    int H;
    // the normalized form's dk (dq = nullptr, no decay, unsplit chains): dden [chains, T] fp32, the
    // gradient of each row's denominator, or nullptr; nk_elu != 0: phi = elu + 1 (else the identity);
    // den [chains, T] fp32, the rows' denominators (required with dden): dout is then the normalized
    // output's gradient do, and the walk's output-gradient role is dn_t = do_t / den_t, formed as each
    // row is staged
    const float *dden;
    int nk_elu;
    const float *den;
};
hipError_t launch_bwd1_bf16(const Bwd1Args &a, hipStream_t s);

}  // namespace la2
