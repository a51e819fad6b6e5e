// rope_vec_kernels.hpp -- the 16-byte vector kernels (in place, out of place,
// several tensors) that read cos/sin tables.
// Included once, by rope_kernels.hip (the one translation unit of the
// library): its kernels are instantiated there, next to the host code
// that selects and launches them.
#pragma once

#include "rope_device.hpp"

namespace rope {
namespace {

// ---------------------------------------------------------------------------
// Vector kernel. A thread works on 16-byte vectors of x: whole interleave
// pairs inside one vector, or rotate_half pairs across two vectors (lanes i
// and i+L/2 in matching positions of vector k of each half).
//
// Tile = one (b,s) position and a chunk of HL*U heads. A block works on GL
// tiles at a time; thread t takes row vector c = lo_vec + t % span, head
// lane hl = (t / span) % HL and tile lane gl = t / (span*HL), and handles
// heads n = chunk*HL*U + hl + k*HL for k < U.
//
// Which vectors a row's threads cover, and who writes what:
// * Interleave: the slice's vectors (lo_vec = start_vec, span = nvec). When
//   the slice covers only part of its first or last 128-byte line, every
//   vector of those lines instead: each line is then requested whole by one
//   wave instruction, which the L2 serves much faster than two half-line
//   requests (it fetches the whole line either way); the vectors outside the
//   slice are loaded and dropped, never stored.
// * rotate_half, pair owner (kModeRH): the threads cover the first half;
//   each loads vector k of both halves and stores both. In place only, for
//   rows whose threads do not fit one wave.
// * rotate_half, own vector (kModeRHOwn): the threads cover the whole slice
//   (or its whole lines, as for interleave); each loads its own vector,
//   takes its partner's (vector k of the other half) from the lane that
//   holds it with ds_bpermute, and stores only its own vector, so each line
//   is requested once by one load instruction and written by one store. The
//   host runs it with single-wave blocks, so a row's threads share a wave:
//   the partner is in reach, and in place the wave's loads have all returned
//   before any of its stores issue, so no thread overwrites a partner's
//   vector before it is read. kModeRHOwnLoad, out of place for rows wider
//   than a wave, loads the partner vector from memory instead.
// * Out of place (src another tensor), the threads cover whole rows:
//   vectors outside the slice are copied from src to x, and every thread
//   stores exactly the vector it covers, with one instruction.
//
// The cos/sin units of a thread are loaded once per tile and, when the
// tables broadcast over heads, reused for all its heads. All loads of a tile
// are issued before any arithmetic. The grid normally has one block per
// group of GL tiles; a smaller grid makes the blocks stride over the groups.
// ---------------------------------------------------------------------------
// x is streamed (each slice byte is read once and written once); the tables
// are re-read by every head and stay in the caches. NT selects nontemporal
// (streaming) loads and stores for x.
template <bool NT>
__device__ __forceinline__ v4u load_x(const v4u* p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void store_x(v4u* p, v4u v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Offsets are 32-bit, in 16-byte vectors for x and in table units for the
// tables: the host runs this kernel only when x spans fewer than 2^32
// vectors (64 GiB) and each table fewer than 2^32 units.
struct VecArgs {
    v4u* x;                 // the tensor written, as 16-byte vectors
    const v4u* src;         // out of place: the tensor read (in place: unused)
    const void* r1;         // cos table, addressed in table units (TableLanes)
    const void* r2;         // sin table
    uint32_t row_vecs;      // vectors per row of x (D*esize/16)
    uint32_t start_vec;     // first slice vector within a row
    uint32_t lo_vec;        // first vector the threads of a row cover
    uint32_t half_vecs;     // rotate_half: x vectors per half of a group (pair distance)
    uint32_t gvec;          // rotate_half: x vectors per group (2*half_vecs; the slice unless a
                            // rotary coefficient splits it into several groups)
    uint32_t thalf;         // rotate_half: table units per half of a group
    uint32_t t1b, t1s, t1n; // cos strides in table units (0 = broadcast)
    uint32_t t2b, t2s, t2n; // sin strides in table units
    uint32_t N;
    uint32_t nvec;          // work units per row (in the slice)
    uint32_t span;          // vectors per row the threads cover (>= nvec)
    uint32_t HL;            // head lanes per tile
    uint32_t GL;            // tiles per block iteration
    uint32_t nchunk;        // head chunks per (b,s)
    uint32_t tiles;         // B*S*nchunk
    uint32_t btiles;        // ceil(tiles / GL)
    uint32_t xcd_group;     // P: runs of P consecutive blocks stay on one XCD
    uint32_t xcd_full;      // blocks [0, xcd_full) are renumbered (a multiple of 8P)
    FastDiv span_div, hl_div, nchunk_div, s_div;  // divisions by span, HL, nchunk, S
    FastDiv xcd_div;        // division by 8P
};

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8), and each XCD has its own L2. The head chunks of one (b,s)
// position are consecutive tiles that read the same table row. Renumber the
// blocks in windows of 8P: within a window, XCD x takes the P consecutive
// tile groups [xP, xP + P). With P a whole number of positions, a table row
// is fetched into one L2 only (dispatch order, P = 1, fetches it into every
// L2), and the 8 XCDs stream through one window of x together. Measured on
// MI355X for a bare whole-line read-modify-write of 1 GiB of 256-byte rows:
// one contiguous eighth of the grid per XCD (P = G/8) was 12% slower than
// dispatch order. The map is a bijection of [0, G); blocks past the last
// whole window keep their number.
__device__ __forceinline__ uint32_t xcd_grouped_block(uint32_t bid, const VecArgs& a)
{
    if (bid >= a.xcd_full) return bid;
    const uint32_t w = fast_div(bid, a.xcd_div);     // window
    const uint32_t l = bid - w * a.xcd_div.d;        // place in the window
    return w * a.xcd_div.d + (l & 7u) * a.xcd_group + (l >> 3);
}

// The 16-byte vector that the lane at byte address `lane4` (lane * 4) of the
// wave holds, through the LDS crossbar (ds_bpermute; no LDS is allocated).
__device__ __forceinline__ v4u lane_exchange(const v4u& v, int lane4)
{
    v4u r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(lane4, (int)v[i]);
    return r;
}

// The kernel body for one tensor: `bid` is the block's number among the G
// blocks that work on this tensor. OUT: read a.src and write a.x (out of
// place); otherwise read and write a.x.
template <int DT, int TT, int DIR, int MODE, int U, bool HEADS_SHARE_TABLES, bool NT, bool OUT>
__device__ __forceinline__ void vec_body(const VecArgs& a, uint32_t bid, uint32_t G)
{
    static_assert(!OUT || MODE != kModeRH, "out of place, rotate_half takes the own-vector scheme");
    constexpr int K = Store<DT>::kLanes;
    using TVec = typename TableLanes<TT, K>::Vec;
    constexpr int TV = TableLanes<TT, K>::kVecs;      // table units per x vector
    static_assert(OUT || MODE != kModeRHOwnLoad, "in place, the own-vector scheme exchanges within the wave");
    constexpr bool kPair = MODE == kModeRH;           // rotate_half, pair owner
    constexpr bool kOwn = MODE == kModeRHOwn || MODE == kModeRHOwnLoad;   // rotate_half, own vector
    constexpr bool kXchg = MODE == kModeRHOwn;        // the partner vector from its lane
    const v4u* src = OUT ? a.src : a.x;
    const TVec* r1 = static_cast<const TVec*>(a.r1);
    const TVec* r2 = static_cast<const TVec*>(a.r2);
    constexpr bool kUnfused = DT != ROPE_DTYPE_F32;
    const uint32_t t = threadIdx.x;
    const uint32_t q = fast_div(t, a.span_div);
    const uint32_t vs = t - q * a.span;
    const uint32_t gl = fast_div(q, a.hl_div);
    const uint32_t hl = q - gl * a.HL;
    // nvec is the slice's vectors (interleave) or half of them (rotate_half).
    // rotate_half pairs vector k of the first half of a group of gvec
    // vectors with vector k of its second half; the slice is one group
    // unless a rotary coefficient splits it.
    const uint32_t rel = a.lo_vec + vs - a.start_vec;  // slice-relative (wraps below the slice)
    const bool in_span = a.lo_vec + vs >= a.start_vec && rel < (kOwn ? 2 * a.nvec : a.nvec);
    // Pair owner: the thread's unit rel is vector k = rel % half_vecs of the
    // first half of group rel / half_vecs.
    const uint32_t c = kPair && a.gvec != 2 * a.nvec
                           ? a.start_vec + (rel / a.half_vecs) * a.gvec + rel % a.half_vecs
                           : a.lo_vec + vs;           // vector within the row
    const uint32_t grel = kOwn && a.gvec != 2 * a.nvec ? rel % a.gvec : rel;   // place in the group
    const bool first = in_span && (!kOwn || grel < a.half_vecs);
    const bool second = kOwn && in_span && grel >= a.half_vecs;
    const bool in_slice = first || second;
    // unit (table index): the first-half vector of the thread's pair
    const uint32_t v = first ? c - a.start_vec : second ? c - a.start_vec - a.half_vecs : 0;
    // Own vector: the partner vector in the other half of the group (outside
    // the slice, the thread's own again), and the table units of the thread's lanes
    // (cos; sin forward) and of the partner's lanes (sin backward).
    const uint32_t partner = first ? c + a.half_vecs : second ? c - a.half_vecs : c;
    const uint32_t t_own = second ? a.thalf : 0;
    const uint32_t t_sin = DIR == kBwd ? (first ? a.thalf : 0) : t_own;
    // Own vector: the partner term is subtracted on the first half forward
    // and on the second half backward.
    const bool neg = DIR == kFwd ? first : second;
    // Own vector, exchange: the byte address of the partner's lane for
    // ds_bpermute (the block is one wave, so the lane is t; the partner is
    // +-half_vecs lanes away in the same row, or the lane itself).
    const int xlane = kXchg ? (int)(t + (partner - c)) * 4 : 0;
    if (gl >= a.GL) return;  // no barriers below, so idle threads may leave

    const uint32_t first_bt = xcd_grouped_block(bid, a);
    for (uint32_t bt = first_bt; bt < a.btiles; bt += G) {
        const uint32_t tile = bt * a.GL + gl;
        if (tile >= a.tiles) continue;
        const uint32_t g = fast_div(tile, a.nchunk_div);  // (b,s) position
        const uint32_t chunk = tile - g * a.nchunk;
        const uint32_t b = fast_div(g, a.s_div);
        const uint32_t s = g - b * a.s_div.d;
        const uint32_t n0 = chunk * (a.HL * U) + hl;
        const uint32_t c_base = b * a.t1b + s * a.t1s + v * TV + (kOwn ? t_own : 0);
        const uint32_t s_base = b * a.t2b + s * a.t2s + v * TV + (kOwn ? t_sin : 0);
        const uint32_t row0 = g * a.N;

        // All loads are issued back to back with no branch between them: a
        // head past N (ragged last chunk) re-reads row N-1 and skips its
        // store. The tables come first, then the x vectors.
        v4u xa[U], xb[U];
        TVec ca[U][TV], sa[U][TV], cb[U][TV], sb[U][TV];
        uint32_t off[U];
        bool live[U];
        if constexpr (HEADS_SHARE_TABLES) {
#pragma unroll
            for (int u = 0; u < TV; ++u) {
                ca[0][u] = r1[c_base + u];
                sa[0][u] = r2[s_base + u];
                if constexpr (kPair) {
                    cb[0][u] = r1[c_base + a.thalf + u];
                    sb[0][u] = r2[s_base + a.thalf + u];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t n = n0 + (uint32_t)k * a.HL;
            live[k] = n < a.N;
            const uint32_t nl = live[k] ? n : a.N - 1;
            const uint32_t row = (row0 + nl) * a.row_vecs;   // the row's first vector
            off[k] = row + c;
            if constexpr (!HEADS_SHARE_TABLES) {
#pragma unroll
                for (int u = 0; u < TV; ++u) {
                    ca[k][u] = r1[c_base + nl * a.t1n + u];
                    sa[k][u] = r2[s_base + nl * a.t2n + u];
                    if constexpr (kPair) {
                        cb[k][u] = r1[c_base + nl * a.t1n + a.thalf + u];
                        sb[k][u] = r2[s_base + nl * a.t2n + a.thalf + u];
                    }
                }
            }
            xa[k] = load_x<NT>(src + off[k]);
            if constexpr (kPair) xb[k] = load_x<NT>(src + off[k] + a.half_vecs);
            if constexpr (kOwn && !kXchg) xb[k] = load_x<NT>(src + row + partner);
        }
        // Keep every load above in flight together: without this barrier the
        // machine scheduler starts the arithmetic on the first vectors and
        // issues the remaining loads only after waiting for them.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kXchg) {
            // every lane of the row takes part (no branch has been taken on
            // the lane's own position yet)
#pragma unroll
            for (int k = 0; k < U; ++k) xb[k] = lane_exchange(xa[k], xlane);
        }

#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (!live[k]) continue;
            if (!OUT && !in_slice) continue;
            // Out of place, a vector outside the slice is copied unchanged.
            // Each vector is stored by one instruction either way, so a
            // 128-byte line that the slice splits is written by one wave
            // instruction rather than two partial ones.
            v4u ya = xa[k], yb = xa[k];
            if (in_slice) {
                const int kt = HEADS_SHARE_TABLES ? 0 : k;
                Lanes<DT> X;
                TableLanes<TT, K> C, S;
                X.unpack(xa[k]);
                C.unpack(ca[kt]);
                S.unpack(sa[kt]);
                if constexpr (MODE == kModeIL) {
#pragma unroll
                    for (int i = 0; i < K; i += 2)
                        rotate_pair<DIR, kUnfused>(X.v[i], X.v[i + 1], C.v[i], S.v[i], C.v[i + 1], S.v[i + 1]);
                } else if constexpr (kPair) {
                    Lanes<DT> X2;
                    TableLanes<TT, K> C2, S2;
                    X2.unpack(xb[k]);
                    C2.unpack(cb[kt]);
                    S2.unpack(sb[kt]);
#pragma unroll
                    for (int i = 0; i < K; ++i)
                        rotate_pair<DIR, kUnfused>(X.v[i], X2.v[i], C.v[i], S.v[i], C2.v[i], S2.v[i]);
                    yb = X2.pack();
                } else {
                    Lanes<DT> P;
                    P.unpack(xb[k]);
#pragma unroll
                    for (int i = 0; i < K; ++i) X.v[i] = rotate_own<kUnfused>(X.v[i], P.v[i], C.v[i], S.v[i], neg);
                }
                ya = X.pack();
            }
            store_x<NT>(a.x + off[k], ya);
            if constexpr (kPair) store_x<NT>(a.x + off[k] + a.half_vecs, yb);
        }
    }
}

template <int DT, int TT, int DIR, int MODE, int U, bool HEADS_SHARE_TABLES, bool NT>
__global__ void __launch_bounds__(256) rope_vec_kernel(VecArgs a)
{
    vec_body<DT, TT, DIR, MODE, U, HEADS_SHARE_TABLES, NT, false>(a, blockIdx.x, gridDim.x);
}

// Out of place: x (the output) receives src with the slice rotated.
template <int DT, int TT, int DIR, int MODE, int U, bool HEADS_SHARE_TABLES, bool NT>
__global__ void __launch_bounds__(256) rope_vec_out_kernel(VecArgs a)
{
    vec_body<DT, TT, DIR, MODE, U, HEADS_SHARE_TABLES, NT, true>(a, blockIdx.x, gridDim.x);
}

// Several tensors that share the tables (the Q and K of one layer) in one
// launch: blocks [first_block[i], first_block[i+1]) work on tensor i. The
// switch keeps every field access a constant offset into the kernel
// arguments.
constexpr int kMultiMax = ROPE_MULTI_MAX;

struct MultiVecArgs {
    uint32_t count;
    uint32_t first_block[kMultiMax + 1];
    VecArgs a[kMultiMax];
};

template <int DT, int TT, int DIR, int MODE, int U, bool HEADS_SHARE_TABLES, bool NT>
__global__ void __launch_bounds__(256) rope_vec_multi_kernel(MultiVecArgs m)
{
    const uint32_t b = blockIdx.x;
    uint32_t i = 0;
#pragma unroll
    for (int k = 1; k < kMultiMax; ++k)
        i += (k < (int)m.count && b >= m.first_block[k]) ? 1u : 0u;
    const uint32_t lo = m.first_block[i], G = m.first_block[i + 1] - lo;
    switch (i) {
    case 0: vec_body<DT, TT, DIR, MODE, U, HEADS_SHARE_TABLES, NT, false>(m.a[0], b - lo, G); break;
    case 1: vec_body<DT, TT, DIR, MODE, U, HEADS_SHARE_TABLES, NT, false>(m.a[1], b - lo, G); break;
    case 2: vec_body<DT, TT, DIR, MODE, U, HEADS_SHARE_TABLES, NT, false>(m.a[2], b - lo, G); break;
    default: vec_body<DT, TT, DIR, MODE, U, HEADS_SHARE_TABLES, NT, false>(m.a[3], b - lo, G); break;
    }
}

}  // namespace
}  // namespace rope
