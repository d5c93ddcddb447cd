// la2_api.cpp -- C ABI of the library: argument checks, work planning, dispatch.
//
// Work decomposition.  Chains (batch x head) are independent: the state a tile
// reads depends only on earlier tiles of the same chain (page "Lightning
// Attention", lizeman.github.io llm-arch-kb, section 2, Step 1).  Each chain is a
// serial walk over its tiles, so when there are fewer chains than compute units
// the sequence is also cut into segments that run on different workgroups:
//   1. a state-only pass gives each segment's own state delta,
//   2. a prefix pass chains the deltas into each segment's start state,
//   3. the output pass runs every segment from its start state.
// With enough chains only step 3 runs, from a zero state.
#include <cstring>
#include <mutex>

#include "la2.h"
#include "la2_internal.h"

namespace {

constexpr int kComputeUnits = 256;   // MI355X: 256 CUs in 8 XCDs

// Plan choices a test can force.  Only the test build of the library (compiled with
// LA2_TEST_HOOKS, exporting la2_test_set_plan) has a way to set them; in the release build they
// are constant zeros, so its launch plan depends on the call's arguments alone.
struct PlanOverride {
    int64_t seg_tiles;      // > 0: tiles per segment of every split chain
    int state_sub;          // > 0: state-pass pieces per segment (used when it divides the segment)
    int slice_width;        // 64: bf16 128-wide values run as two 64-wide slices
    int separate_dkdv;      // != 0: the two separate reverse scans instead of the fused dk/dv pass
    int64_t norm_segment;   // > 0: positions per segment of the denominator scans
    int two_pass_backward;  // != 0: la2_backward_saved without decay by the dQ pass and the dK/dV pass
    int legacy_forward;     // != 0: forward-direction bf16 output passes on the 8-wave scan kernel only
    int legacy_dkdv;        // != 0: the fused dk/dv pass on its 8-wave kernel only
    int reverse_prefix;     // != 0: the reverse prefix launch even where the backward walk would sum the
                            //   deltas of its later pieces itself
};

#ifdef LA2_TEST_HOOKS
PlanOverride g_override{};
const PlanOverride &forced() { return g_override; }
#else
constexpr PlanOverride kNoOverride{};
constexpr const PlanOverride &forced() { return kNoOverride; }
#endif

struct Plan {
    int TB;          // tile length the kernels run with
    int nseg;        // segments per chain
    int seg_tiles;   // tiles per segment
    int sub;         // state-pass sub-segments per segment (sub divides seg_tiles)
    int nsub;        // state entries per chain (sub-segments of seg_tiles / sub tiles)
    int narrow;      // bf16: run 128-wide value tensors as two 64-wide slices
    size_t ws_bytes; // workspace for the segment states
};

// Sub-segments of the state-only pass.  It has (nseg - 1) segments per chain to sum, one workgroup
// each, and one workgroup fills a CU, so with few chains it can leave CUs idle (128 chains split
// in two: half the chip).  Cutting each segment into `sub` pieces (at least 32 tiles each, so the
// extra fp32 state written per piece stays small next to the tiles it sums) gives more workgroups;
// sub is chosen to fill whole rounds of the 256 CUs best, and only when that gains 10%.
// `most` caps the pieces per segment (the no-alloc forward's states must fit its static scratch).
int choose_sub(int64_t work, int nseg, int seg_tiles, int64_t most) {
    if (nseg < 2) return 1;
    if (const int v = forced().state_sub; v > 0) return seg_tiles % v == 0 ? v : 1;
    const int64_t base = work * (nseg - 1);
    auto fill = [&](int r) {
        const int64_t w = base * r, rounds = (w + kComputeUnits - 1) / kComputeUnits;
        return (double)w / (double)(rounds * kComputeUnits);
    };
    int best = 1;
    double bf = fill(1);
    for (int r = 2; seg_tiles / r >= 32 && r <= most; ++r)
        if (seg_tiles % r == 0 && fill(r) > bf + 0.1) {
            best = r;
            bf = fill(r);
        }
    return best;
}

int elem_size(int dtype) { return dtype == LA2_BF16 ? 2 : 4; }

// Tile lengths a caller may ask for (page "Lightning Attention", section 2: ceil(T / T_B) tiles of
// any length; section 4 sweeps 64, 128 and 256).
bool block_ok(int block) { return block == 16 || block == 32 || block == 64 || block == 128 || block == 256; }

// Tile length the output kernels run for a requested `block`.  The intra/inter split is exact for
// every tile length, so the request is met by the nearest length a kernel is built for: bf16 tiles
// are 64 or 128 positions (32-row MFMA blocks; a 256 tile's Q, K and V alone would fill LDS), fp32
// tiles 16, 32 or 64.
int run_tile(int dtype, int block) {
    if (dtype == LA2_BF16) return block < 64 ? 64 : block > 128 ? 128 : block;
    return block > 64 ? 64 : block;
}

// Value-slice width a kernel launch uses for a value tensor of width `w`.
int slice_width(int dtype, int w, int narrow) { return dtype == LA2_BF16 ? (narrow ? 64 : w) : 64; }

int check_sizes(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dv, int block, int dtype) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || dv <= 0) return LA2_ERR_BAD_SHAPE;
    // every byte offset must fit comfortably in int64, and grid dimensions in 32 bits
    const int64_t lim = (int64_t)1 << 40;
    if (B > lim / H) return LA2_ERR_BAD_SHAPE;
    const int64_t chains = B * H;
    if (chains > (int64_t)1 << 24 || T > lim / chains || chains * T > lim / 512) return LA2_ERR_BAD_SHAPE;
    if (!((d == 64 || d == 128) && (dv == 64 || dv == 128))) return LA2_ERR_UNSUPPORTED;
    if (!block_ok(block)) return LA2_ERR_UNSUPPORTED;
    return LA2_OK;
}

// `fused`: the plan of the fused bf16 dk/dv pass, which tiles by kDkdvTile and splits only T.
// `cap`: most workspace bytes the plan may need (the state-pass pieces are limited to fit); without
// forced choices, one piece per segment always fits 16 MiB (at most 256 segment states of
// d x d_v <= 128 x 128 fp32).
Plan make_plan(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dv, int block, int dtype, bool fused = false,
               size_t cap = SIZE_MAX) {
    Plan p{};
    p.TB = fused ? la2::kDkdvTile : run_tile(dtype, block);
    const int64_t NT = (T + p.TB - 1) / p.TB;
    const int64_t chains = B * H;
    // Too few chains to fill the chip: split T into segments (one extra state pass over k and v,
    // whose result the backward reuses).  Running a 128-wide value as two 64-wide slices would
    // avoid that pass (the kernel's XCD-aware order serves both slices' q and k from one L2), but
    // each slice still forms the whole score block, about 0.6 of a full slice's work, and measured
    // slower than segments once the backward reuses the forward's states; only a forced plan uses it.
    p.narrow = !fused && dtype == LA2_BF16 && dv == 128 && forced().slice_width == 64;
    const int64_t slices = dv / slice_width(dtype, (int)dv, p.narrow);
    const int64_t work = chains * slices;
    int64_t seg_tiles = NT;
    if (const int64_t v = forced().seg_tiles; v > 0) {
        seg_tiles = v < NT ? v : NT;
    } else if (!p.narrow && work < kComputeUnits && NT > 1) {
        int64_t nseg = kComputeUnits / work;
        if (nseg > NT) nseg = NT;
        seg_tiles = (NT + nseg - 1) / nseg;
    }
    p.seg_tiles = (int)seg_tiles;
    p.nseg = (int)((NT + seg_tiles - 1) / seg_tiles);
    const size_t per_piece = (size_t)chains * p.nseg * d * dv * sizeof(float);
    p.sub = choose_sub(work, p.nseg, p.seg_tiles, (int64_t)(cap / per_piece));
    const int64_t sub_tiles = seg_tiles / p.sub;
    p.nsub = p.nseg > 1 ? (int)((NT + sub_tiles - 1) / sub_tiles) : 1;
    p.ws_bytes = p.nseg > 1 ? (size_t)chains * p.nsub * d * dv * sizeof(float) : 0;
    return p;
}

// The backward computes dk and dv in one fused pass where a kernel exists for the shape (bf16,
// d = d_v), else by two separate reverse scans.
bool fused_dkdv(int64_t d, int64_t dv, int dtype) {
    return dtype == LA2_BF16 && la2::dkdv_supported((int)d, (int)dv) && !forced().separate_dkdv;
}

// Shapes whose training step without decay runs the one-pass backward (la2_bwd1_bf16.hip).
bool bwd1_shape(int64_t d, int64_t dv, int dtype) {
    return dtype == LA2_BF16 && d == 128 && dv == 128 && !forced().separate_dkdv && !forced().two_pass_backward;
}

// Plan of the one-pass backward: the forward plan's segments (whose start states it reads), cut into
// kBwd1Tile-position tiles; sub / nsub / ws_bytes describe its reverse state pass.
Plan bwd1_plan(const Plan &fwd, int64_t chains, int64_t T, int64_t d, int64_t dv) {
    Plan p{};
    p.TB = la2::kBwd1Tile;
    p.nseg = fwd.nseg;
    p.seg_tiles = fwd.seg_tiles * (fwd.TB / la2::kBwd1Tile);
    p.sub = choose_sub(chains, p.nseg, p.seg_tiles, INT32_MAX);
    const int64_t sub_tiles = p.seg_tiles / p.sub;
    const int64_t nt = (T + p.TB - 1) / p.TB;
    p.nsub = p.nseg > 1 ? (int)((nt + sub_tiles - 1) / sub_tiles) : 1;
    p.ws_bytes = p.nseg > 1 ? (size_t)chains * p.nsub * d * dv * sizeof(float) : 0;
    return p;
}

// Backward workspace: [S segment states, exactly as la2_forward leaves them][each chain's final state
// (shapes of the one-pass backward only), which la2_forward leaves there when given this much
// workspace and no decay][R segment states].  Keeping the forward's states in place lets
// la2_backward_saved skip recomputing them.
size_t backward_ws_bytes(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dv, int block, int dtype,
                         size_t *s_bytes = nullptr, size_t *f_bytes = nullptr) {
    const Plan pl = make_plan(B, H, T, d, dv, block, dtype);
    const size_t a = pl.ws_bytes;
    size_t b = fused_dkdv(d, dv, dtype) ? make_plan(B, H, T, d, dv, block, dtype, true).ws_bytes : a;
    size_t f = 0;
    if (bwd1_shape(d, dv, dtype)) {
        f = (size_t)(B * H) * d * dv * sizeof(float);
        const size_t r = bwd1_plan(pl, B * H, T, d, dv).ws_bytes;
        if (r > b) b = r;
    }
    if (s_bytes) *s_bytes = a;
    if (f_bytes) *f_bytes = f;
    return a + f + b;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};

Range range_of(const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

la2::ScanArgs scan_args(const void *a, const void *b, const void *c, void *y, const float *decay, int64_t chains,
                        int64_t H, int64_t T, int W, const Plan &pl, int dtype) {
    la2::ScanArgs args{};
    args.a = a;
    args.b = b;
    args.c = c;
    args.y = y;
    args.decay = decay;
    args.T = T;
    args.H = (int)H;
    args.DVT = W;
    args.nseg = pl.nseg;
    args.seg_tiles = pl.seg_tiles;
    args.chains = (int)chains;
    args.nslice = W / slice_width(dtype, W, pl.narrow);
    args.sub = pl.sub;
    args.nsub = pl.nsub;
    return args;
}

hipError_t launch(const la2::ScanArgs &args, int D, const Plan &pl, int dtype, la2::Dir dir, la2::Mode mode,
                  hipStream_t s) {
    const int DV = slice_width(dtype, args.DVT, pl.narrow);
    if (dtype == LA2_BF16 && mode == la2::Mode::StateOnly) return la2::launch_state_bf16(args, D, DV, pl.TB, dir, s);
    if (dtype == LA2_BF16 && mode == la2::Mode::Output && dir == la2::Dir::Forward && !forced().legacy_forward &&
        D == 128 && DV == 128 && args.nslice == 1 && !args.den && !args.has_init) {
        // at d = d_v = 128: the producer/consumer scan over 64-position tiles
        la2::Fwd1Args f{};
        f.q = args.a;
        f.k = args.b;
        f.v = args.c;
        f.y = args.y;
        f.T = args.T;
        f.seg_len = (int64_t)args.seg_tiles * pl.TB;
        f.nseg = args.nseg;
        f.chains = args.chains;
        f.states = args.nseg > 1 ? args.states : nullptr;
        f.states_t = args.states_t;
        f.sub = args.sub;
        f.nsub = args.nsub;
        f.state_out = args.state_out;
        f.decay = args.decay;
        f.H = args.H;
        return la2::launch_fwd1_bf16(f, s);
    }
    return dtype == LA2_BF16 ? la2::launch_scan_bf16(args, D, DV, pl.TB, dir, s)
                             : la2::launch_scan_f32(args, D, DV, pl.TB, dir, mode, s);
}

// Segment start states of the scan with key role `b` (width D) and value role `c` (width W) in
// direction `dir`, written to `ws` ([chains, nseg, D, W] fp32).  Only called for split chains.
// `init` ([chains, D, W] or nullptr): the state the first segment starts from.
// compose (and no init): leave the state pass's per-piece deltas in `ws` without the prefix launch, for
// an output kernel that sums them itself.
// A walk that sums the reverse deltas itself reads each later piece's 64 KiB at its start (four
// memory round trips per piece before its first tile) instead of one prefix launch for all (~10 us):
// 10 us faster at two pieces, no faster at 5-15 pieces.
constexpr int kComposeMaxPieces = 2;
bool compose_reverse(const Plan &p) {
    return p.nseg > 1 && !forced().reverse_prefix && p.nsub - 1 - la2::state_index(0, p.sub, p.nsub, true) <= kComposeMaxPieces;
}

int segment_states(const void *b, const void *c, const float *decay, int64_t chains, int64_t H, int64_t T, int D,
                   int W, const Plan &pl, int dtype, la2::Dir dir, void *ws, hipStream_t s,
                   const float *init = nullptr, bool compose = false) {
    // the state pass runs the sub-segments: every state entry is one segment of its own
    Plan sp = pl;
    sp.seg_tiles = pl.seg_tiles / pl.sub;
    sp.nseg = pl.nsub;
    sp.sub = 1;
    la2::ScanArgs args = scan_args(nullptr, b, c, nullptr, decay, chains, H, T, W, sp, dtype);
    args.states = static_cast<float *>(ws);
    // deltas of the sub-segments that some later (forward) / earlier (reverse) output segment needs
    args.seg_first = dir == la2::Dir::Forward ? 0 : pl.sub;
    args.seg_count = dir == la2::Dir::Forward ? (pl.nseg - 1) * pl.sub : pl.nsub - pl.sub;
    if (launch(args, D, sp, dtype, dir, la2::Mode::StateOnly, s) != hipSuccess) return LA2_ERR_HIP;
    if (compose && init == nullptr) return LA2_OK;
    // a reverse init sits at the chain's last position: the last piece's length - 1 before its start
    const int64_t init_len = T - 1 - (int64_t)(pl.nsub - 1) * sp.seg_tiles * pl.TB;
    if (la2::launch_segment_prefix(args.states, decay, (int)chains, (int)H, pl.nsub, (int64_t)sp.seg_tiles * pl.TB,
                                   (int64_t)D * W, dir, s, init, init_len) != hipSuccess)
        return LA2_ERR_HIP;
    return LA2_OK;
}

// Output pass y = attention(a, b, c) in direction `dir`, every segment starting from the states in
// `ws` (transposed when states_t) or from zero when the chains are not split.  `state_in`
// ([chains, D, W], read transposed when states_t) is where an unsplit chain starts (a split chain's
// first segment in scan order reads it from `ws`, where the prefix put it): forward, a carried-in
// state; reverse, the gradient of a carried-out state.  `state_out` receives the forward's final
// state, or in reverse lam times the state at position 0.
int output_scan(const void *a, const void *b, const void *c, void *y, const float *decay, int64_t chains, int64_t H,
                int64_t T, int D, int W, const Plan &pl, int dtype, la2::Dir dir, void *ws, int states_t,
                hipStream_t s, const float *state_in = nullptr, float *state_out = nullptr,
                const float *den = nullptr) {
    la2::ScanArgs args = scan_args(a, b, c, y, decay, chains, H, T, W, pl, dtype);
    args.den = den;
    args.states = pl.nseg > 1 ? static_cast<float *>(ws) : const_cast<float *>(state_in);
    args.has_init = state_in != nullptr;
    args.state_out = state_out;
    args.states_t = states_t;
    args.seg_first = 0;
    args.seg_count = pl.nseg;
    return launch(args, D, pl, dtype, dir, la2::Mode::Output, s) == hipSuccess ? LA2_OK : LA2_ERR_HIP;
}

}  // namespace

extern "C" {

int la2_abi_version(void) { return LA2_ABI_VERSION; }

#ifdef LA2_TEST_HOOKS
int la2_test_set_plan(int64_t seg_tiles, int state_sub, int slice_width, int separate_dkdv, int64_t norm_segment,
                      int two_pass_backward, int legacy_forward, int legacy_dkdv, int reverse_prefix) {
    g_override = PlanOverride{seg_tiles,      state_sub,   slice_width, separate_dkdv, norm_segment,
                              two_pass_backward, legacy_forward, legacy_dkdv, reverse_prefix};
    return LA2_OK;
}
#endif

const char *la2_status_string(int status) {
    switch (status) {
        case LA2_OK: return "ok";
        case LA2_ERR_NULL_POINTER: return "a required pointer is NULL";
        case LA2_ERR_BAD_SHAPE: return "B, H, T, d and d_v must be positive and the tensors addressable";
        case LA2_ERR_UNSUPPORTED: return "d, d_v, block or dtype outside the compiled set";
        case LA2_ERR_MISALIGNED: return "tensor pointers must be 16-byte aligned";
        case LA2_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
        case LA2_ERR_WORKSPACE_TOO_SMALL: return "workspace missing or smaller than la2_workspace_bytes";
        case LA2_ERR_HIP: return "HIP kernel launch failed";
        case LA2_ERR_SCRATCH_TOO_SMALL:
            return "the sizes need more segment-state scratch than the static buffer of la2_forward_noalloc holds";
        default: return "unknown status";
    }
}

size_t la2_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype,
                           int backward) {
    if (check_sizes(B, H, T, d, d_v, block, dtype) != LA2_OK) return (size_t)-1;
    return backward ? backward_ws_bytes(B, H, T, d, d_v, block, dtype) : make_plan(B, H, T, d, d_v, block, dtype).ws_bytes;
}

}  // extern "C"

namespace {

// `den` (fp32 [B, H, T] or nullptr): o_t is divided by den_t before it is stored (the normalized form).
int forward_impl(const void *q, const void *k, const void *v, const float *decay, const float *state_in, void *o,
                 float *state_out, int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype,
                 void *workspace, size_t workspace_bytes, void *stream, const float *den = nullptr,
                 size_t cap = SIZE_MAX, bool train_final = false) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return LA2_ERR_NULL_POINTER;
    int st = check_sizes(B, H, T, d, d_v, block, dtype);
    if (st != LA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (workspace && !aligned16(workspace)) ||
        !aligned16(state_in) || !aligned16(state_out) || (reinterpret_cast<uintptr_t>(decay) & 3u))
        return LA2_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)(B * H * T * d) * es, nv = (size_t)(B * H * T * d_v) * es;
    const size_t ns = (size_t)(B * H * d * d_v) * sizeof(float);
    const Plan pl = make_plan(B, H, T, d, d_v, block, dtype, false, cap);
    const Range ro = range_of(o, nv);
    const Range rdec = range_of(decay, decay ? (size_t)H * 4 : 0);
    const Range rsi = range_of(state_in, state_in ? ns : 0), rso = range_of(state_out, state_out ? ns : 0);
    if (overlap(ro, range_of(q, nq)) || overlap(ro, range_of(k, nq)) || overlap(ro, range_of(v, nv)) ||
        overlap(ro, rdec) || overlap(ro, rsi) || overlap(ro, rso))
        return LA2_ERR_ALIAS;
    // the final state may overwrite the initial one in place, but may not partly overlap it or any input
    if (state_out && ((overlap(rso, rsi) && state_out != state_in) || overlap(rso, range_of(q, nq)) ||
                      overlap(rso, range_of(k, nq)) || overlap(rso, range_of(v, nv)) || overlap(rso, rdec)))
        return LA2_ERR_ALIAS;
    if (pl.ws_bytes) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return LA2_ERR_WORKSPACE_TOO_SMALL;
        const Range rw = range_of(workspace, pl.ws_bytes);
        if (overlap(rw, ro) || overlap(rw, range_of(q, nq)) || overlap(rw, range_of(k, nq)) ||
            overlap(rw, range_of(v, nv)) || overlap(rw, rdec) || overlap(rw, rsi) || overlap(rw, rso))
            return LA2_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t chains = B * H;
    // Given room for the backward (and no decay), the forward also leaves each chain's final state in the
    // workspace, where the one-pass backward of la2_backward_saved starts from it.
    if (train_final && !state_out && !decay && bwd1_shape(d, d_v, dtype) && workspace) {
        size_t a = 0, f = 0;
        if (workspace_bytes >= backward_ws_bytes(B, H, T, d, d_v, block, dtype, &a, &f))
            state_out = reinterpret_cast<float *>(static_cast<char *>(workspace) + a);
    }
    if (pl.nseg > 1) {
        st = segment_states(k, v, decay, chains, H, T, (int)d, (int)d_v, pl, dtype, la2::Dir::Forward, workspace, s,
                            state_in);
        if (st != LA2_OK) return st;
    }
    return output_scan(q, k, v, o, decay, chains, H, T, (int)d, (int)d_v, pl, dtype, la2::Dir::Forward, workspace,
                       0, s, state_in, state_out, den);
}

}  // namespace

extern "C" {

int la2_forward(const void *q, const void *k, const void *v, const float *decay, void *o, int64_t B, int64_t H,
                int64_t T, int64_t d, int64_t d_v, int block, int dtype, void *workspace, size_t workspace_bytes,
                void *stream) {
    return forward_impl(q, k, v, decay, nullptr, o, nullptr, B, H, T, d, d_v, block, dtype, workspace,
                        workspace_bytes, stream, nullptr, SIZE_MAX, true);
}

int la2_forward_state(const void *q, const void *k, const void *v, const float *decay, const float *state_in,
                      void *o, float *state_out, int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block,
                      int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(q, k, v, decay, state_in, o, state_out, B, H, T, d, d_v, block, dtype, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of la2_forward_noalloc: the segment states of split chains, in a static device array that
// each GPU the library runs on holds until the process ends.  Host code never uses the array's name
// as an address (on the host it names a stand-in, not device memory): each device's address is
// looked up once, with that device current, and kept.
constexpr size_t kScratchBytes = LA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (hipGetDevice), looked up on its first use.
int current_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LA2_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LA2_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LA2_OK;
}

}  // namespace

extern "C" {

int la2_forward_noalloc(const void *q, const void *k, const void *v, const float *decay, void *o, int64_t B,
                        int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype, void *stream) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return LA2_ERR_NULL_POINTER;
    const int st = check_sizes(B, H, T, d, d_v, block, dtype);
    if (st != LA2_OK) return st;
    const size_t need = make_plan(B, H, T, d, d_v, block, dtype, false, kScratchBytes).ws_bytes;
    if (need > kScratchBytes) return LA2_ERR_SCRATCH_TOO_SMALL;
    void *ws = nullptr;
    if (need > 0) {
        const int sst = current_scratch(&ws);
        if (sst != LA2_OK) return sst;
    }
    // every segment state the prefix reads is written by the state pass first: nothing to clear
    return forward_impl(q, k, v, decay, nullptr, o, nullptr, B, H, T, d, d_v, block, dtype, ws,
                        need > 0 ? kScratchBytes : 0, stream, nullptr, kScratchBytes);
}

int la2_decode_step(const void *q, const void *k, const void *v, const float *decay, void *o, float *state,
                    int64_t B, int64_t H, int64_t d, int64_t d_v, int dtype, void *stream) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o || !state) return LA2_ERR_NULL_POINTER;
    const int st = check_sizes(B, H, 1, d, d_v, dtype == LA2_BF16 ? 128 : 64, dtype);
    if (st != LA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state) ||
        (reinterpret_cast<uintptr_t>(decay) & 3u))
        return LA2_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)(B * H * d) * es, nv = (size_t)(B * H * d_v) * es;
    const Range ro = range_of(o, nv), rs = range_of(state, (size_t)(B * H * d * d_v) * sizeof(float));
    const Range rdec = range_of(decay, decay ? (size_t)H * 4 : 0);
    const Range ins[4] = {range_of(q, nq), range_of(k, nq), range_of(v, nv), rdec};
    for (const Range &r : ins)
        if (overlap(ro, r) || overlap(rs, r)) return LA2_ERR_ALIAS;
    if (overlap(ro, rs)) return LA2_ERR_ALIAS;
    return la2::launch_decode(q, k, v, decay, o, state, (int)(B * H), (int)H, (int)d, (int)d_v, dtype,
                              static_cast<hipStream_t>(stream)) == hipSuccess
               ? LA2_OK
               : LA2_ERR_HIP;
}

int la2_forward_serial(const void *q, const void *k, const void *v, const float *decay, void *o, int64_t B, int64_t H,
                       int64_t T, int64_t d, int64_t d_v, int dtype, void *stream) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return LA2_ERR_NULL_POINTER;
    const int st = check_sizes(B, H, T, d, d_v, dtype == LA2_BF16 ? 128 : 64, dtype);
    if (st != LA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (reinterpret_cast<uintptr_t>(decay) & 3u))
        return LA2_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)(B * H * T * d) * es, nv = (size_t)(B * H * T * d_v) * es;
    const Range ro = range_of(o, nv);
    const Range ins[4] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                          range_of(decay, decay ? (size_t)H * 4 : 0)};
    for (const Range &r : ins)
        if (overlap(ro, r)) return LA2_ERR_ALIAS;
    return la2::launch_serial(q, k, v, decay, o, (int)(B * H), (int)H, T, (int)d, (int)d_v, dtype,
                              static_cast<hipStream_t>(stream)) == hipSuccess
               ? LA2_OK
               : LA2_ERR_HIP;
}

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Segments of the denominator pass: enough (chain, segment) workgroups to give every compute unit
// about 8, each segment at least 256 positions and a multiple of the kernel's 64-position chunk.
struct DenPlan {
    int64_t seg_len;
    int nseg;
};

DenPlan den_plan(int64_t chains, int64_t T) {
    int64_t nseg = 1;
    if (chains < 8 * kComputeUnits) {
        nseg = (8 * kComputeUnits + chains - 1) / chains;
        const int64_t most = (T + 255) / 256;
        if (nseg > most) nseg = most;
    }
    int64_t seg_len = (T + nseg - 1) / nseg;
    if (const int64_t v = forced().norm_segment; v > 0) seg_len = v;
    seg_len = (seg_len + 63) / 64 * 64;
    return DenPlan{seg_len, (int)((T + seg_len - 1) / seg_len)};
}

// Workspace of the normalized forward: [phi(q)][phi(k)] (elu + 1 only), [den, fp32 per position],
// [segment sums of the denominator's vector scans] (split chains only), [the numerator scan's own
// workspace]; the backward takes the numerator backward's workspace in the same place (its first
// part holds the states exactly as the numerator forward leaves them) and adds [dden, fp32 per
// position][dn, the numerator's output gradient][the reverse segment sums of its dk part] after it,
// so everything the forward wrote sits where the backward reads it and nothing overwrites it
// (la2_backward_normalized_saved may run again on the same workspace).  Every part 256-byte aligned.
struct NormLayout {
    size_t phi;        // bytes of each of phi(q), phi(k)
    size_t den_off, dden_off, dn_off;
    size_t z_off, z_bytes, y_off;
    size_t scan_off, scan_bytes;
    // bf16 backward only (dq from the centered feature map, la2_norm.hip mode 7): the per-segment
    // sums of phi(k) for its mean m, phi(k) - m, the scan U of (dout, v, phi(k) - m) and that scan's
    // segment states, a_t = dout_t . (prefix sum of v)_t and the segment sums of v
    size_t m_off, kap_off, u_off, a_off, vz_off, us_off, us_bytes;
    size_t total;
    DenPlan dp;
};

NormLayout norm_layout(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dv, int fmap, int block, int dtype,
                       bool backward = false) {
    NormLayout L{};
    const int64_t chains = B * H;
    const size_t rows_f32 = align256((size_t)(chains * T) * sizeof(float));
    L.phi = fmap ? align256((size_t)(chains * T * d) * elem_size(dtype)) : 0;
    L.dp = den_plan(chains, T);
    L.den_off = 2 * L.phi;
    L.z_off = L.den_off + rows_f32;
    L.z_bytes = L.dp.nseg > 1 ? align256((size_t)chains * L.dp.nseg * d * sizeof(float)) : 0;
    L.scan_off = L.z_off + L.z_bytes;
    L.scan_bytes = align256(backward ? backward_ws_bytes(B, H, T, d, dv, block, dtype)
                                     : make_plan(B, H, T, d, dv, block, dtype).ws_bytes);
    L.dden_off = L.scan_off + L.scan_bytes;
    L.dn_off = L.dden_off + (backward ? rows_f32 : 0);
    L.y_off = L.dn_off + (backward ? align256((size_t)(chains * T * dv) * elem_size(dtype)) : 0);
    L.total = L.y_off + (backward ? L.z_bytes : 0);
    if (backward && dtype == LA2_BF16) {
        const size_t tile_bytes = align256((size_t)(chains * T * d) * elem_size(dtype));
        L.m_off = L.total;
        L.kap_off = L.m_off + align256((size_t)chains * L.dp.nseg * d * sizeof(float));
        L.u_off = L.kap_off + tile_bytes;
        L.a_off = L.u_off + tile_bytes;
        L.vz_off = L.a_off + rows_f32;
        L.us_off = L.vz_off + (L.dp.nseg > 1 ? align256((size_t)chains * L.dp.nseg * dv * sizeof(float)) : 0);
        L.us_bytes = align256(make_plan(B, H, T, d, dv, block, dtype).ws_bytes);
        L.total = L.us_off + L.us_bytes;
    }
    return L;
}

la2::DenArgs den_args(const void *q, const void *k, const float *decay, char *ws, const NormLayout &L, int64_t H,
                      int64_t T, int64_t chains) {
    la2::DenArgs a{};
    a.q = q;
    a.k = k;
    a.pq = L.phi ? ws : nullptr;
    a.pk = L.phi ? ws + L.phi : nullptr;
    a.den = reinterpret_cast<float *>(ws + L.den_off);
    a.decay = decay;
    a.zseg = L.z_bytes ? reinterpret_cast<float *>(ws + L.z_off) : nullptr;
    a.T = T;
    a.seg_len = L.dp.seg_len;
    a.H = (int)H;
    a.nseg = L.dp.nseg;
    a.chains = (int)chains;
    return a;
}

// Scan modes of launch_vscan (la2_norm.hip).
constexpr int kVZSeg = 0, kVDen = 1, kVDQ = 2, kVYSeg = 3, kVDK = 4, kVMean = 5, kVKappa = 6, kVDQN = 7;

// The normalized forward as one launch of the 64-position producer/consumer scan (la2_fwd1_bf16.hip):
// bf16 at d = d_v = 128 without decay, on chains the plan does not split.
bool fused_normalized(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dv, int block, int dtype,
                      const float *decay) {
    if (dtype != LA2_BF16 || d != 128 || dv != 128 || decay || forced().legacy_forward) return false;
    const Plan pl = make_plan(B, H, T, d, dv, block, dtype);
    return pl.nseg == 1 && slice_width(dtype, (int)dv, pl.narrow) == dv;
}

// o, and where given phi(q), phi(k) (elu + 1 only), the denominators and the sums of phi(k) over the
// denominator plan's segments (msum, for the bf16 backward's mean), of the fused normalized forward.
hipError_t launch_fused_normalized(const void *q, const void *k, const void *v, void *o, void *pq, void *pk,
                                   float *den, float *msum, int64_t msum_seg, int64_t chains, int64_t T,
                                   int feature_map, hipStream_t s) {
    la2::Fwd1Args f{};
    f.q = q;
    f.k = k;
    f.v = v;
    f.y = o;
    f.T = T;
    f.seg_len = (T + 63) / 64 * 64;
    f.nseg = 1;
    f.chains = (int)chains;
    f.sub = f.nsub = 1;
    f.norm = feature_map == LA2_PHI_ELU1 ? 2 : 1;
    f.pq = pq;
    f.pk = pk;
    f.den = den;
    f.msum = msum;
    f.msum_seg = msum_seg;
    return la2::launch_fwd1_bf16(f, s);
}

}  // namespace

extern "C" {

size_t la2_normalized_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int feature_map,
                                      int block, int dtype, int backward) {
    if (check_sizes(B, H, T, d, d_v, block, dtype) != LA2_OK || (feature_map != 0 && feature_map != 1))
        return (size_t)-1;
    return norm_layout(B, H, T, d, d_v, feature_map, block, dtype, backward != 0).total;
}

int la2_forward_normalized(const void *q, const void *k, const void *v, const float *decay, void *o, int64_t B,
                           int64_t H, int64_t T, int64_t d, int64_t d_v, int feature_map, int block, int dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (feature_map != LA2_PHI_IDENTITY && feature_map != LA2_PHI_ELU1) return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return LA2_ERR_NULL_POINTER;
    int st = check_sizes(B, H, T, d, d_v, block, dtype);
    if (st != LA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (workspace && !aligned16(workspace)) ||
        (reinterpret_cast<uintptr_t>(decay) & 3u))
        return LA2_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)(B * H * T * d) * es, nv = (size_t)(B * H * T * d_v) * es;
    const NormLayout L = norm_layout(B, H, T, d, d_v, feature_map, block, dtype);
    const Range ins[4] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                          range_of(decay, decay ? (size_t)H * 4 : 0)};
    const Range ro = range_of(o, nv);
    for (const Range &r : ins)
        if (overlap(ro, r)) return LA2_ERR_ALIAS;
    if (L.total) {
        if (!workspace || workspace_bytes < L.total) return LA2_ERR_WORKSPACE_TOO_SMALL;
        const Range rw = range_of(workspace, L.total);
        if (overlap(rw, ro)) return LA2_ERR_ALIAS;
        for (const Range &r : ins)
            if (overlap(rw, r)) return LA2_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const int64_t chains = B * H;
    // bf16 at d = d_v = 128 without decay, chains the plan does not split: one launch applies phi to
    // the tiles and forms numerator and denominator together.  Given room for the backward it also
    // leaves phi(q), phi(k), the denominators and each denominator segment's plain sum of phi(k) (the
    // bf16 backward's mean) where la2_backward_normalized_saved reads them, and (denominator segments of
    // split chains) each segment's sum of phi(k), which the bf16 dq carries.
    if (fused_normalized(B, H, T, d, d_v, block, dtype, decay)) {
        const NormLayout LB = norm_layout(B, H, T, d, d_v, feature_map, block, dtype, true);
        const bool for_bwd = workspace && workspace_bytes >= LB.total;
        if (launch_fused_normalized(q, k, v, o, for_bwd && L.phi ? ws : nullptr, for_bwd && L.phi ? ws + L.phi : nullptr,
                                    for_bwd ? reinterpret_cast<float *>(ws + L.den_off) : nullptr,
                                    for_bwd ? reinterpret_cast<float *>(ws + LB.m_off) : nullptr, LB.dp.seg_len, chains,
                                    T, feature_map, s) != hipSuccess)
            return LA2_ERR_HIP;
        if (for_bwd && L.dp.nseg > 1 &&
            la2::launch_vscan(den_args(q, k, decay, ws, L, H, T, chains), (int)d, dtype, feature_map, kVZSeg, s) !=
                hipSuccess)
            return LA2_ERR_HIP;
        return LA2_OK;
    }
    // 1. denominator den_t = phi(q_t) . z_t (fp32), and phi(q), phi(k) for the numerator
    const la2::DenArgs a = den_args(q, k, decay, ws, L, H, T, chains);
    if (a.nseg > 1 && la2::launch_vscan(a, (int)d, dtype, feature_map, kVZSeg, s) != hipSuccess) return LA2_ERR_HIP;
    if (la2::launch_vscan(a, (int)d, dtype, feature_map, kVDen, s) != hipSuccess) return LA2_ERR_HIP;
    // 2. numerator: the plain scan on phi(q), phi(k), each output row divided by its den_t before it is
    //    stored (in fp32, so o is rounded once)
    return forward_impl(L.phi ? a.pq : q, L.phi ? a.pk : k, v, decay, nullptr, o, nullptr, B, H, T, d, d_v, block,
                        dtype, L.scan_bytes ? ws + L.scan_off : nullptr, L.scan_bytes, stream, a.den);
}

}  // extern "C"

namespace {

// Where the normalized backward's dK/dV walk takes the denominator's part of dk and forms dn = do / den
// itself: bf16, d = d_v = 128, no decay, chains the dK/dV plan does not split.
bool nk_walk(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dv, int block, int dtype, const float *decay) {
    if (dtype != LA2_BF16 || d != 128 || dv != 128 || decay || forced().legacy_dkdv || !fused_dkdv(d, dv, dtype))
        return false;
    return make_plan(B, H, T, d, dv, block, dtype, true).nseg == 1;
}

// reuse_s: the S segment states that la2_forward left at the start of the workspace are still there.
// nk_dden, nk_den (the normalized form's backward, with skip_dq, where nk_walk holds): the rows'
// denominator gradients and denominators; dout is then do, and the dK/dV walk forms dn = do / den,
// adds the denominator's part of dk and the feature map's derivative (nk_elu: elu + 1, else the
// identity) and sets *nk_done.
int backward_impl(const void *q, const void *k, const void *v, const float *decay, const void *dout, void *dq,
                  void *dk, void *dv, int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream, bool reuse_s, const float *state_in = nullptr,
                  const float *dstate_out = nullptr, float *dstate_in = nullptr, bool one_pass = false,
                  bool skip_dq = false, const float *nk_dden = nullptr, bool nk_elu = false,
                  bool *nk_done = nullptr, const float *nk_den = nullptr) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    // dout given as do rather than dn: only the walk that divides it may run
    if ((nk_den != nullptr) != (nk_dden != nullptr) ||
        (nk_den && (!skip_dq || state_in || dstate_out || dstate_in || !nk_walk(B, H, T, d, d_v, block, dtype, decay))))
        return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !dout || (!dq && !skip_dq) || !dk || !dv) return LA2_ERR_NULL_POINTER;
    int st = check_sizes(B, H, T, d, d_v, block, dtype);
    if (st != LA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv) || (workspace && !aligned16(workspace)) || (reinterpret_cast<uintptr_t>(decay) & 3u) ||
        !aligned16(state_in) || !aligned16(dstate_out) || !aligned16(dstate_in))
        return LA2_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)(B * H * T * d) * es, nv = (size_t)(B * H * T * d_v) * es;
    const size_t ns = (size_t)(B * H * d * d_v) * sizeof(float);
    const Plan pl = make_plan(B, H, T, d, d_v, block, dtype);
    const bool fused = fused_dkdv(d, d_v, dtype);
    size_t s_bytes = 0, f_bytes = 0;
    const size_t ws_need = backward_ws_bytes(B, H, T, d, d_v, block, dtype, &s_bytes, &f_bytes);
    const Range ins[7] = {range_of(q, nq), range_of(k, nq), range_of(v, nv), range_of(dout, nv),
                          range_of(decay, decay ? (size_t)H * 4 : 0), range_of(state_in, state_in ? ns : 0),
                          range_of(dstate_out, dstate_out ? ns : 0)};
    const Range outs[5] = {range_of(dq, skip_dq ? 0 : nq), range_of(dk, nq), range_of(dv, nv),
                           range_of(workspace, ws_need), range_of(dstate_in, dstate_in ? ns : 0)};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlap(outs[i], ins[j])) return LA2_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return LA2_ERR_ALIAS;
    }
    if (ws_need && (!workspace || workspace_bytes < ws_need)) return LA2_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t chains = B * H;
    const int D = (int)d, DV = (int)d_v;
    st = LA2_OK;
    const bool split = pl.nseg > 1;
    void *ws_r = workspace ? static_cast<char *>(workspace) + s_bytes + f_bytes : nullptr;
    if (one_pass && !skip_dq && reuse_s && !decay && !state_in && !dstate_out && !dstate_in &&
        bwd1_shape(d, d_v, dtype)) {
        // Training step without decay: dq, dk and dv in one reverse walk from the forward's segment start
        // states and final states (left in the workspace), and the reverse states at the segment ends.
        const Plan bp = bwd1_plan(pl, chains, T, d, d_v);
        if (bp.nseg > 1 && (st = segment_states(q, dout, nullptr, chains, H, T, D, DV, bp, dtype, la2::Dir::Reverse,
                                                ws_r, s, nullptr, compose_reverse(bp))) != LA2_OK)
            return st;
        la2::Bwd1Args a{};
        a.q = q;
        a.k = k;
        a.v = v;
        a.dout = dout;
        a.dq = dq;
        a.dk = dk;
        a.dv = dv;
        a.T = T;
        a.nseg = bp.nseg;
        a.seg_tiles = bp.seg_tiles;
        a.chains = (int)chains;
        a.s_states = split ? static_cast<const float *>(workspace) : nullptr;
        a.s_sub = pl.sub;
        a.s_nsub = pl.nsub;
        a.s_final = reinterpret_cast<const float *>(static_cast<const char *>(workspace) + s_bytes);
        a.r_states = bp.nseg > 1 ? static_cast<const float *>(ws_r) : nullptr;
        a.r_sub = bp.sub;
        a.r_nsub = bp.nsub;
        a.r_compose = compose_reverse(bp);
        a.r_piece_len = (int64_t)(bp.seg_tiles / bp.sub) * bp.TB;
        return la2::launch_bwd1_bf16(a, s) == hipSuccess ? LA2_OK : LA2_ERR_HIP;
    }
    // dq_t = S_t do_t          = forward scan with (query, key, value) = (do, v, k); its state is S^T, so
    // it reads the forward's S states ([d, d_v] per segment) transposed
    if (!skip_dq) {
        if (split && !reuse_s &&
            (st = segment_states(k, v, decay, chains, H, T, D, DV, pl, dtype, la2::Dir::Forward, workspace, s,
                                 state_in)) != LA2_OK)
            return st;
        if ((st = output_scan(dout, v, k, dq, decay, chains, H, T, DV, D, pl, dtype, la2::Dir::Forward, workspace, 1,
                              s, state_in)) != LA2_OK)
            return st;
    }
    if (fused) {
        // dk_t = R_t v_t and dv_t = R_t^T k_t in one reverse pass, R_t = lam R_{t+1} + q_t do_t^T
        const Plan fp = make_plan(B, H, T, d, d_v, block, dtype, true);
        // d = d_v = 128, no carried state: the walk, which sums the reverse deltas itself
        const bool walk = d == 128 && d_v == 128 && !dstate_out && !dstate_in && !forced().legacy_dkdv;
        if (fp.nseg > 1 && (st = segment_states(q, dout, decay, chains, H, T, D, DV, fp, dtype, la2::Dir::Reverse,
                                                ws_r, s, dstate_out, walk && compose_reverse(fp))) != LA2_OK)
            return st;
        if (walk) {
            // d = d_v = 128, no carried state: the producer/consumer walk of the one-pass backward without
            // its dQ and S (la2_bwd1_bf16.hip), R from the reverse states at the segment ends
            la2::Bwd1Args a{};
            a.q = q;
            a.k = k;
            a.v = v;
            a.dout = dout;
            a.dk = dk;
            a.dv = dv;
            a.T = T;
            a.nseg = fp.nseg;
            a.seg_tiles = fp.seg_tiles;
            a.chains = (int)chains;
            a.r_states = fp.nseg > 1 ? static_cast<const float *>(ws_r) : nullptr;
            a.r_sub = fp.sub;
            a.r_nsub = fp.nsub;
            a.r_compose = compose_reverse(fp);
            a.r_piece_len = (int64_t)(fp.seg_tiles / fp.sub) * fp.TB;
            a.decay = decay;
            a.H = (int)H;
            if (nk_dden && skip_dq && !decay && fp.nseg == 1) {
                a.dden = nk_dden;
                a.den = nk_den;
                a.nk_elu = nk_elu ? 1 : 0;
                if (nk_done) *nk_done = true;
            }
            return la2::launch_bwd1_bf16(a, s) == hipSuccess ? LA2_OK : LA2_ERR_HIP;
        }
        la2::DkdvArgs a{};
        a.q = q;
        a.k = k;
        a.v = v;
        a.dout = dout;
        a.dk = dk;
        a.dv = dv;
        a.decay = decay;
        a.states = fp.nseg > 1 ? static_cast<const float *>(ws_r) : dstate_out;
        a.has_init = dstate_out != nullptr;
        a.state_out = dstate_in;
        a.T = T;
        a.H = (int)H;
        a.nseg = fp.nseg;
        a.seg_tiles = fp.seg_tiles;
        a.chains = (int)chains;
        a.sub = fp.sub;
        a.nsub = fp.nsub;
        return la2::launch_dkdv_bf16(a, D, s) == hipSuccess ? LA2_OK : LA2_ERR_HIP;
    }
    // reverse state R_t = lam R_{t+1} + q_t do_t^T, [d, d_v], shared by the dv and dk scans
    if (split && (st = segment_states(q, dout, decay, chains, H, T, D, DV, pl, dtype, la2::Dir::Reverse, ws_r, s,
                                      dstate_out)) != LA2_OK)
        return st;
    // dv_t = R_t^T k_t         = reverse scan with (k, q, do), state R; it also gives lam R_0
    if ((st = output_scan(k, q, dout, dv, decay, chains, H, T, D, DV, pl, dtype, la2::Dir::Reverse, ws_r, 0, s,
                          dstate_out, dstate_in)) != LA2_OK)
        return st;
    // dk_t = R_t v_t           = reverse scan with (v, do, q), state R^T: read R transposed
    return output_scan(v, dout, q, dk, decay, chains, H, T, DV, D, pl, dtype, la2::Dir::Reverse, ws_r, 1, s,
                       dstate_out);
}

}  // namespace

extern "C" {

int la2_backward(const void *q, const void *k, const void *v, const float *decay, const void *dout, void *dq,
                 void *dk, void *dv, int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype,
                 void *workspace, size_t workspace_bytes, void *stream) {
    return backward_impl(q, k, v, decay, dout, dq, dk, dv, B, H, T, d, d_v, block, dtype, workspace, workspace_bytes,
                         stream, false);
}

int la2_backward_saved(const void *q, const void *k, const void *v, const float *decay, const void *dout, void *dq,
                       void *dk, void *dv, int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block,
                       int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return backward_impl(q, k, v, decay, dout, dq, dk, dv, B, H, T, d, d_v, block, dtype, workspace, workspace_bytes,
                         stream, true, nullptr, nullptr, nullptr, true);
}

int la2_backward_state(const void *q, const void *k, const void *v, const float *decay, const float *state_in,
                       const void *dout, const float *dstate_out, void *dq, void *dk, void *dv, float *dstate_in,
                       int64_t B, int64_t H, int64_t T, int64_t d, int64_t d_v, int block, int dtype, void *workspace,
                       size_t workspace_bytes, void *stream) {
    return backward_impl(q, k, v, decay, dout, dq, dk, dv, B, H, T, d, d_v, block, dtype, workspace, workspace_bytes,
                         stream, false, state_in, dstate_out, dstate_in);
}

}  // extern "C"

namespace {

// saved: phi(q), phi(k), the denominators, their segment sums and the numerator's segment states are
// still in the workspace from la2_forward_normalized on the same inputs.
int backward_normalized_impl(const void *q, const void *k, const void *v, const float *decay, const void *o,
                             const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t T,
                             int64_t d, int64_t d_v, int feature_map, int block, int dtype, void *workspace,
                             size_t workspace_bytes, void *stream, bool saved) {
    if (dtype != LA2_F32 && dtype != LA2_BF16) return LA2_ERR_UNSUPPORTED;
    if (feature_map != LA2_PHI_IDENTITY && feature_map != LA2_PHI_ELU1) return LA2_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o || !dout || !dq || !dk || !dv) return LA2_ERR_NULL_POINTER;
    int st = check_sizes(B, H, T, d, d_v, block, dtype);
    if (st != LA2_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || (workspace && !aligned16(workspace)) ||
        (reinterpret_cast<uintptr_t>(decay) & 3u))
        return LA2_ERR_MISALIGNED;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)(B * H * T * d) * es, nv = (size_t)(B * H * T * d_v) * es;
    const NormLayout L = norm_layout(B, H, T, d, d_v, feature_map, block, dtype, true);
    if (!workspace || workspace_bytes < L.total) return LA2_ERR_WORKSPACE_TOO_SMALL;
    const Range ins[6] = {range_of(q, nq), range_of(k, nq), range_of(v, nv), range_of(o, nv), range_of(dout, nv),
                          range_of(decay, decay ? (size_t)H * 4 : 0)};
    const Range outs[4] = {range_of(dq, nq), range_of(dk, nq), range_of(dv, nv), range_of(workspace, L.total)};
    for (int i = 0; i < 4; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r)) return LA2_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return LA2_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const int64_t chains = B * H;
    la2::DenArgs a = den_args(q, k, decay, ws, L, H, T, chains);
    float *dden = reinterpret_cast<float *>(ws + L.dden_off);
    void *dn = ws + L.dn_off;
    // 1. the forward's denominator, phi(q), phi(k) (recomputed unless the forward left them), the way the
    //    forward forms them: where it is one fused launch, that launch again, its o put in dn's place
    //    (overwritten next)
    if (!saved) {
        if (fused_normalized(B, H, T, d, d_v, block, dtype, decay)) {
            if (launch_fused_normalized(q, k, v, dn, a.pq, a.pk, a.den, reinterpret_cast<float *>(ws + L.m_off),
                                        L.dp.seg_len, chains, T, feature_map, s) != hipSuccess ||
                (a.nseg > 1 && la2::launch_vscan(a, (int)d, dtype, feature_map, kVZSeg, s) != hipSuccess))
                return LA2_ERR_HIP;
        } else {
            if (a.nseg > 1 && la2::launch_vscan(a, (int)d, dtype, feature_map, kVZSeg, s) != hipSuccess)
                return LA2_ERR_HIP;
            if (la2::launch_vscan(a, (int)d, dtype, feature_map, kVDen, s) != hipSuccess) return LA2_ERR_HIP;
        }
    }
    const bool centered = dtype == LA2_BF16;
    // where the dK/dV walk takes the denominator's dk it also forms dn = do / den as it stages each tile,
    // and the centered dq combination writes dden: no pass over o
    const bool nk = centered && nk_walk(B, H, T, d, d_v, block, dtype, decay);
    // 2. dn = do / den, dden = -(do . o) / den
    if (!nk && la2::launch_grad_rows(o, dout, a.den, dn, dden, chains * T, (int)d_v, dtype, s) != hipSuccess)
        return LA2_ERR_HIP;
    if (centered) {
        // bf16: dq of the centered feature map (la2_norm.hip, mode 7), every step in fp32 except the scan U
        // of (dout, v, phi(k) - m), whose values are small against the result
        la2::DenArgs c = a;
        c.msum = reinterpret_cast<float *>(ws + L.m_off);
        c.kap = ws + L.kap_off;
        // where the forward is one fused launch: the segment sums of phi(k) for its mean are the
        // forward's (any constant m makes the rewrite exact, so they may come from phi(k) rounded to
        // bf16), and U's scan forms kap = phi(k) - m from k on chip (its chains are unsplit too)
        const bool fused = fused_normalized(B, H, T, d, d_v, block, dtype, decay);
        if (!fused && (la2::launch_vscan(c, (int)d, dtype, feature_map, kVMean, s) != hipSuccess ||
                       la2::launch_vscan(c, (int)d, dtype, feature_map, kVKappa, s) != hipSuccess))
            return LA2_ERR_HIP;
        // a_t = dout_t . Vbar_t: the denominator scan with (query, key) = (dout, v) and the identity map
        // (where the scan U below is one fused launch, that launch forms it as its rows' sums)
        la2::DenArgs va = c;
        va.q = dout;
        va.k = v;
        va.pq = va.pk = nullptr;
        va.den = reinterpret_cast<float *>(ws + L.a_off);
        va.zseg = L.dp.nseg > 1 ? reinterpret_cast<float *>(ws + L.vz_off) : nullptr;
        if (!fused && ((va.nseg > 1 && la2::launch_vscan(va, (int)d_v, dtype, 0, kVZSeg, s) != hipSuccess) ||
                       la2::launch_vscan(va, (int)d_v, dtype, 0, kVDen, s) != hipSuccess))
            return LA2_ERR_HIP;
        // U = the forward scan with (query, key, value) = (dout, v, phi(k) - m), as the dQ pass of the
        // plain backward: its state is (sum kap v^T)^T
        if (fused) {
            la2::Fwd1Args f{};
            f.q = dout;
            f.k = v;
            f.v = k;
            f.y = ws + L.u_off;
            f.den = va.den;   // a_t
            f.T = T;
            f.seg_len = (T + 63) / 64 * 64;
            f.nseg = 1;
            f.chains = (int)chains;
            f.sub = f.nsub = 1;
            f.norm = feature_map == LA2_PHI_ELU1 ? 4 : 3;
            f.msum = c.msum;
            f.msum_seg = L.dp.seg_len;
            if (la2::launch_fwd1_bf16(f, s) != hipSuccess) return LA2_ERR_HIP;
        } else {
            const Plan pl = make_plan(B, H, T, d, d_v, block, dtype);
            void *uws = L.us_bytes ? ws + L.us_off : nullptr;
            if (pl.nseg > 1 && (st = segment_states(c.kap, v, decay, chains, H, T, (int)d, (int)d_v, pl, dtype,
                                                    la2::Dir::Forward, uws, s)) != LA2_OK)
                return st;
            if ((st = output_scan(dout, v, c.kap, ws + L.u_off, decay, chains, H, T, (int)d_v, (int)d, pl, dtype,
                                  la2::Dir::Forward, uws, 1, s)) != LA2_OK)
                return st;
        }
        c.u = ws + L.u_off;
        c.arow = va.den;
        c.g = dq;
        c.dden_out = nk ? dden : nullptr;
        if (la2::launch_vscan(c, (int)d, dtype, feature_map, kVDQN, s) != hipSuccess) return LA2_ERR_HIP;
    }
    // 3. the numerator's gradients: the plain backward on (phi(q), phi(k), v) with output gradient dn;
    //    dv is final, dq (fp32 only) and dk hold the gradients with respect to phi(q), phi(k) so far --
    //    except where the dK/dV walk runs on unsplit chains (nk): there it reads do and den for dn, also
    //    takes dden and returns the final dk
    bool nk_done = false;
    st = backward_impl(L.phi ? a.pq : q, L.phi ? a.pk : k, v, decay, nk ? dout : dn, centered ? nullptr : dq, dk, dv,
                       B, H, T, d, d_v, block, dtype, L.scan_bytes ? ws + L.scan_off : nullptr, L.scan_bytes, stream,
                       saved, nullptr, nullptr, nullptr, false, centered, nk ? dden : nullptr,
                       feature_map == LA2_PHI_ELU1, &nk_done, nk ? a.den : nullptr);
    if (st != LA2_OK) return st;
    // 4. the denominator's: dq_t += dden_t z_t (the forward segment sums of phi(k) are still in place; fp32
    //    only), dk_t += sum_{s >= t} lam^(s-t) dden_s phi(q_s); then the feature map's derivative
    a.dden = dden;
    a.g = dq;
    if (!centered && la2::launch_vscan(a, (int)d, dtype, feature_map, kVDQ, s) != hipSuccess) return LA2_ERR_HIP;
    if (nk_done) return LA2_OK;
    a.g = dk;
    a.zseg = L.z_bytes ? reinterpret_cast<float *>(ws + L.y_off) : nullptr;   // the forward's z sums stay
    if (a.nseg > 1 && la2::launch_vscan(a, (int)d, dtype, feature_map, kVYSeg, s) != hipSuccess) return LA2_ERR_HIP;
    return la2::launch_vscan(a, (int)d, dtype, feature_map, kVDK, s) == hipSuccess ? LA2_OK : LA2_ERR_HIP;
}

}  // namespace

extern "C" {

int la2_backward_normalized(const void *q, const void *k, const void *v, const float *decay, const void *o,
                            const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t T, int64_t d,
                            int64_t d_v, int feature_map, int block, int dtype, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return backward_normalized_impl(q, k, v, decay, o, dout, dq, dk, dv, B, H, T, d, d_v, feature_map, block, dtype,
                                    workspace, workspace_bytes, stream, false);
}

int la2_backward_normalized_saved(const void *q, const void *k, const void *v, const float *decay, const void *o,
                                  const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t T,
                                  int64_t d, int64_t d_v, int feature_map, int block, int dtype, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return backward_normalized_impl(q, k, v, decay, o, dout, dq, dk, dv, B, H, T, d, d_v, feature_map, block, dtype,
                                    workspace, workspace_bytes, stream, true);
}

}  // extern "C"
