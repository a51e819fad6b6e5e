// Partial rotary position embedding for MI355X (gfx950, CDNA4), in place
// and out of place.
//
// Operation: "CANN ops-transformer 算子详解：inplace_partial_rotary_mul
// 原地部分旋转位置编码", section 功能与计算公式 (interleave pairs (2i,2i+1),
// out = x*cos + x_rotate*sin on the lanes [start,end), in place) and section
// 自动微分说明 (backward = gradient w.r.t. x); rotate_half pairs (i, i+L/2)
// from "ANE实战RoPE位置编码在MIL中的纯ANE实现", section 先搞懂RoPE.
// Precision: the mixed-precision paragraph of the first page's tiling/kernel
// section -- 16-bit data is computed in fp32 and written back with
// round-to-nearest-even.
//
// The page's AICore kernel builds an XOR-1 gather table, multiplies, gathers,
// negates the even lanes with a bit mask and adds, in separate vector passes.
// Here a thread instead loads whole rotation pairs with 16-byte loads (a pair
// of 16-bit lanes is one 32-bit word; a pair of fp32 lanes is 8 bytes), does
// the swap and sign in registers, computes in fp32 (one fp32 rounding, exact
// products for 16-bit data) and stores only the slice's 16-byte vectors, so
// lanes outside [start,end) are never written (in place). The path is
// HBM-bound (0.375-0.75 flop per byte), so there is no MFMA and nothing is
// staged in LDS (rotate_half partners may move between lanes through the LDS
// crossbar, ds_bpermute): a block takes a chunk of heads of one (b,s)
// position, the blocks of a position run on one XCD, and when the tables
// broadcast over heads its cos/sin rows are fetched from HBM once and served
// by that XCD's L2 to every head.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <string>

#include "rope_fastdiv.hpp"
#include "rope_partial.h"
#include "rope_plan.hpp"

namespace rope {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // one 16-byte vector
typedef uint32_t v2u __attribute__((ext_vector_type(2)));  // half of one

constexpr int kModeRH = ROPE_MODE_ROTATE_HALF;
constexpr int kModeIL = ROPE_MODE_INTERLEAVE;
// rotate_half schemes of the vector kernel (see there): each thread writes
// its own vector and takes its partner's from the lane that holds it (a
// row's threads in one wave), or loads the partner from memory (out of
// place, rows wider than a wave)
constexpr int kModeRHOwn = 2;
constexpr int kModeRHOwnLoad = 3;

// ---------------------------------------------------------------------------
// fp32 <-> storage conversions. A 32-bit word holds two adjacent 16-bit lanes
// (lower lane in the low half). Widening is exact; narrowing rounds to nearest
// even (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32), keeps fp16 subnormals and
// NaNs, and overflows to infinity.
// ---------------------------------------------------------------------------
template <int DT> struct Store;

template <> struct Store<ROPE_DTYPE_BF16> {
    static constexpr int kLanes = 8;  // per 16-byte vector
    __device__ static f32x2 widen(uint32_t w)
    {
        f32x2 r;
        r.x = __uint_as_float(w << 16);
        r.y = __uint_as_float(w & 0xffff0000u);
        return r;
    }
    __device__ static uint32_t narrow(f32x2 v)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
    __device__ static float load1(const void* p, int64_t i)
    {
        return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
    }
    __device__ static void store1(void* p, int64_t i, float v)
    {
        static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
};

template <> struct Store<ROPE_DTYPE_F16> {
    static constexpr int kLanes = 8;
    __device__ static f32x2 widen(uint32_t w)
    {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    }
    __device__ static uint32_t narrow(f32x2 v)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
    __device__ static float load1(const void* p, int64_t i)
    {
        return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    }
    __device__ static void store1(void* p, int64_t i, float v)
    {
        static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
    }
};

template <> struct Store<ROPE_DTYPE_F32> {
    static constexpr int kLanes = 4;
    __device__ static float load1(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
    __device__ static void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};

// A 16-byte vector of lanes as fp32 values.
template <int DT>
struct Lanes {
    float v[Store<DT>::kLanes];
    __device__ void unpack(const v4u& q)
    {
        if constexpr (DT == ROPE_DTYPE_F32) {
            v[0] = __uint_as_float(q[0]); v[1] = __uint_as_float(q[1]);
            v[2] = __uint_as_float(q[2]); v[3] = __uint_as_float(q[3]);
        } else {
            const uint32_t w[4] = {q[0], q[1], q[2], q[3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f32x2 f = Store<DT>::widen(w[k]);
                v[2 * k] = f.x;
                v[2 * k + 1] = f.y;
            }
        }
    }
    __device__ v4u pack() const
    {
        if constexpr (DT == ROPE_DTYPE_F32) {
            return v4u{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                       __float_as_uint(v[3])};
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f32x2 f;
                f.x = v[2 * k];
                f.y = v[2 * k + 1];
                w[k] = Store<DT>::narrow(f);
            }
            return v4u{w[0], w[1], w[2], w[3]};
        }
    }
};

// ---------------------------------------------------------------------------
// The rotation of one pair (a, b) = (x_j, x_p(j)) where j is the lane whose
// partner term is negated in the forward (even lane / first half):
//   forward : a' = a*c_a - b*s_a        b' = b*c_b + a*s_b
//   backward: a' = a*c_a + b*s_b        b' = b*c_b - a*s_a   (transpose)
// 16-bit x (UNFUSED): each product is rounded to fp32 and the sum is rounded
// once more, as the page's "cast to fp32, multiply-add in fp32" reads. With
// 16-bit tables both products are exact, so this is also the single
// rounding of the exact sum; with fp32 tables the product roundings are part
// of the definition. fp32 x: the compiler may fuse (the result is held to a
// tolerance, not to bits).
// ---------------------------------------------------------------------------
template <int DIR>
__device__ __forceinline__ void rotate_pair_unfused(float& a, float& b, float ca, float sa, float cb, float sb)
{
#pragma clang fp contract(off)
    // no fused multiply-add in this function: every product and sum rounds
    float na, nb;
    if constexpr (DIR == kFwd) {
        na = a * ca - b * sa;
        nb = b * cb + a * sb;
    } else {
        na = a * ca + b * sb;
        nb = b * cb - a * sa;
    }
    a = na;
    b = nb;
}

template <int DIR, bool UNFUSED>
__device__ __forceinline__ void rotate_pair(float& a, float& b, float ca, float sa, float cb, float sb)
{
    if constexpr (UNFUSED) {
        rotate_pair_unfused<DIR>(a, b, ca, sa, cb, sb);
    } else {
        float na, nb;
        if constexpr (DIR == kFwd) {
            na = a * ca - b * sa;
            nb = b * cb + a * sb;
        } else {
            na = a * ca + b * sb;
            nb = b * cb - a * sa;
        }
        a = na;
        b = nb;
    }
}

// One lane of rotate_half in the own-vector scheme: the lane's value x, its
// partner's value p, and y = x*c - p*s (neg) or x*c + p*s, with c the lane's
// cos and s the sine the direction takes (the lane's forward, the partner's
// backward). These are the same products and sum as rotate_pair forms for
// that lane, with the same roundings.
__device__ __forceinline__ float rotate_own_unfused(float x, float p, float c, float s, bool neg)
{
#pragma clang fp contract(off)
    const float t = p * s;
    return x * c + (neg ? -t : t);
}

template <bool UNFUSED>
__device__ __forceinline__ float rotate_own(float x, float p, float c, float s, bool neg)
{
    if constexpr (UNFUSED) {
        return rotate_own_unfused(x, p, c, s, neg);
    } else {
        const float t = p * s;
        return x * c + (neg ? -t : t);
    }
}

// The cos or sin values for the K lanes of one x vector, from a table of
// type TT. They take K * sizeof(TT) bytes, loaded as kVecs table units of
// type Vec: 8 bytes (half a vector) when fp32 x meets a 16-bit table, one
// 16-byte vector when the table is as wide as x, two when 16-bit x meets an
// fp32 table (the page's mixed bf16-x / fp32-table case).
template <int Bytes> struct TableUnit { using type = v4u; };
template <> struct TableUnit<8> { using type = v2u; };

template <int TT, int K>
struct TableLanes {
    static constexpr int kBytes = K * (TT == ROPE_DTYPE_F32 ? 4 : 2);
    static_assert(kBytes == 8 || kBytes == 16 || kBytes == 32, "table unit shape");
    using Vec = typename TableUnit<kBytes>::type;
    static constexpr int kVecs = kBytes == 32 ? 2 : 1;
    float v[K];
    __device__ void unpack(const Vec* q)
    {
        if constexpr (TT == ROPE_DTYPE_F32) {
#pragma unroll
            for (int t = 0; t < kVecs; ++t)
#pragma unroll
                for (int w = 0; w < 4; ++w) v[4 * t + w] = __uint_as_float(q[t][w]);
        } else {
#pragma unroll
            for (int w = 0; w < kBytes / 4; ++w) {
                f32x2 f = Store<TT>::widen(q[0][w]);
                v[2 * w] = f.x;
                v[2 * w + 1] = f.y;
            }
        }
    }
};

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

// ---------------------------------------------------------------------------
// cos and sin from positions ("ANE实战RoPE位置编码在MIL中的纯ANE实现", section
// 第一步: the table of θ = p / base^(2i/h), here θ = p * inv_freq[i] with the
// frequencies given): θ is the double product of the position and the pair's
// frequency, cos θ and sin θ are evaluated in double precision and rounded
// once, to nearest even, to the table type TT.
// ---------------------------------------------------------------------------

// A double rounded once to the nearest value of TT, ties to even, returned
// as the float that holds it. fp32: the conversion instruction (round to
// nearest even). bf16/fp16: a value of the type is a whole number of units
// in the last place of its binade, 2^(e - p) for |v| in [2^(e-1), 2^e) with
// p significand bits, and never below the least subnormal 2^(emin - p + 1);
// scaling by powers of two is exact and rint() rounds ties to even.
template <int TT>
__device__ __forceinline__ float round_to_type(double v)
{
    if constexpr (TT == ROPE_DTYPE_F32) {
        return static_cast<float>(v);
    } else {
        constexpr int p = TT == ROPE_DTYPE_F16 ? 11 : 8;
        constexpr int emin = TT == ROPE_DTYPE_F16 ? -14 : -126;
        constexpr double maxf = TT == ROPE_DTYPE_F16 ? 65504.0 : 0x1.fep127;
        if (!(v != 0.0) || !__builtin_isfinite(v)) return static_cast<float>(v);   // zero, inf, NaN
        int e;
        (void)frexp(v, &e);
        const int q = e - p > emin - p + 1 ? e - p : emin - p + 1;
        const double r = ldexp(rint(ldexp(v, -q)), q);
        if (fabs(r) > maxf) return v > 0 ? __builtin_inff() : -__builtin_inff();
        return static_cast<float>(r);   // exact: r is a value of TT
    }
}

// (cos θ, sin θ) rounded to TT for position p and frequency f.
template <int TT>
__device__ __forceinline__ float2 pos_cos_sin(int64_t p, double f)
{
    double sn, cn;
    sincos(static_cast<double>(p) * f, &sn, &cn);
    return make_float2(round_to_type<TT>(cn), round_to_type<TT>(sn));
}

// ---------------------------------------------------------------------------
// Vector kernel with the tables computed from positions. A block takes P
// consecutive (b,s) positions (P > 1 only when one position's heads fill
// fewer than kPosLanes threads) and, for each, a chunk of up to HL*kUPos
// heads (HL head lanes, kUPos heads per thread). Its threads first load the
// position and frequency of the first (cos, sin) pair each evaluates, then
// issue their x loads, then evaluate cos and sin while x is in flight: the
// memory counter drains in issue order, so the wait for the frequency does
// not wait for x, provided every load is issued on every path (indices are
// clamped, never branched around). The values go to LDS, each pair of each
// position once per block, and each thread reads those of its lanes from
// there. The thread layout is the table kernel's: interleave with
// whole-line coverage, rotate_half as pair owner (a thread takes vector k
// of both halves). Measured on MI355X (the (16,8192,32,128) shard's slice
// [32,96), the GQA Q layout at 4096 positions, the MLA-style slice): two
// heads per thread in 128-thread blocks was the best of 1, 2, 4 or 8 heads
// per thread in 64-, 128- or 256-thread blocks on all three, and as fast as
// the table kernel on the first two.
// ---------------------------------------------------------------------------
constexpr int kUPos = 2;
constexpr int kPosLds = ROPE_D_LIMIT / 2;    // (cos, sin) entries per block
constexpr uint32_t kPosLanes = 128;          // threads a position's heads fill before a block takes more positions
// The out-of-place position kernel's heads per thread and threads per
// position, by mode. Measured on MI355X (cold data; the (16,8192,32,128)
// shard's lanes [32,96), the MLA-style slice, a whole rotate_half head and
// its second half), over 1, 2 or 4 heads per thread in blocks of 64, 128 or
// 256 threads: interleave was fastest with 2 heads in 128 threads (326 and
// 257 us), rotate_half with 4 heads in 64 threads (165 and 164 us, the table
// path's times; 172 and 167 us with the interleave shape).
constexpr int pos_out_heads(int mode) { return mode == kModeIL ? 2 : 4; }
constexpr uint32_t pos_out_lanes(int mode) { return mode == kModeIL ? 128 : 64; }

struct PosArgs {
    v4u* x;                  // the tensor written (in place: also read)
    const v4u* src;          // out of place: the tensor read
    const int64_t* pos;      // position of (b,s) at pos[b*pos_sb + s*pos_ss]
    const double* inv_freq;  // L/2 frequencies
    int64_t pos_sb, pos_ss;
    uint32_t row_vecs;       // vectors per row of x
    uint32_t start_vec;      // first slice vector within a row
    uint32_t lo_vec;         // first vector the threads of a row cover
    uint32_t half_vecs;      // rotate_half: vectors per half of a group (pair distance)
    uint32_t gvec;           // rotate_half: vectors per group (2*half_vecs)
    uint32_t nvec;           // work units per row (interleave: slice vectors; rotate_half: half of them)
    uint32_t span;           // vectors per row the threads cover
    uint32_t HL;             // head lanes per position
    uint32_t lanes;          // threads per position: span * HL
    uint32_t P;              // positions per block
    uint32_t N;
    uint32_t pairs;          // L/2
    uint32_t entries;        // P * pairs
    uint32_t chunks;         // head chunks per position
    uint32_t bs;             // B*S
    uint32_t items;          // ceil(B*S / P) * chunks
    FastDiv span_div, lanes_div, pairs_div, chunk_div, s_div;
    // Several tensors in one launch (MULTI): N counts the heads of all of
    // them; head n of a position belongs to the last tensor q with
    // hoff[q] <= n (hoff past the last tensor is UINT32_MAX), which holds
    // nt[q] heads per position and starts at xs[q].
    v4u* xs[kMultiMax];
    uint32_t nt[kMultiMax];
    uint32_t hoff[kMultiMax];
};

// The row of head nl of position g in one tensor, or, MULTI, in the tensor
// the head belongs to; as a vector pointer with the thread's vector c.
template <bool MULTI>
__device__ __forceinline__ v4u* pos_row_vec(const PosArgs& a, uint32_t g, uint32_t nl, uint32_t c)
{
    if constexpr (!MULTI) {
        return a.x + ((g * a.N + nl) * a.row_vecs + c);
    } else {
        v4u* base = a.xs[0];
        uint32_t nt = a.nt[0], ho = 0;
#pragma unroll
        for (int q = 1; q < kMultiMax; ++q) {
            const bool in = nl >= a.hoff[q];
            base = in ? a.xs[q] : base;
            nt = in ? a.nt[q] : nt;
            ho = in ? a.hoff[q] : ho;
        }
        return base + ((g * nt + (nl - ho)) * a.row_vecs + c);
    }
}

template <int DT, int TT, int DIR, int MODE, bool MULTI>
__global__ void __launch_bounds__(256) rope_pos_kernel(PosArgs a)
{
    __shared__ float2 cs[kPosLds];   // (cos, sin) of the block's positions, pair-major per position
    constexpr int K = Store<DT>::kLanes;
    constexpr int U = kUPos;
    constexpr bool kUnfused = DT != ROPE_DTYPE_F32;
    const uint32_t t = threadIdx.x;
    const uint32_t pp = fast_div(t, a.lanes_div);   // the thread's position within the block
    const uint32_t r = t - pp * a.lanes;
    const uint32_t hl = fast_div(r, a.span_div);
    const uint32_t vs = r - hl * a.span;
    const uint32_t c = a.lo_vec + vs;                 // vector within the row
    const bool in_slice = c >= a.start_vec && c - a.start_vec < a.nvec;
    const uint32_t v = in_slice ? c - a.start_vec : 0;
    // rotate_half: unit v is vector v % half_vecs of the first half of group
    // v / half_vecs (one group unless a rotary coefficient splits the slice);
    // its lanes are pairs v*K + e either way
    const uint32_t cx = MODE == kModeRH && a.gvec != 2 * a.nvec
                            ? a.start_vec + (v / a.half_vecs) * a.gvec + v % a.half_vecs
                            : c;
    // the table entry this thread evaluates first: position eq, pair ei
    const uint32_t eq = fast_div(t, a.pairs_div);
    const uint32_t ei = t - eq * a.pairs;
    // every thread runs the same iterations, so the barriers below are uniform
    for (uint32_t w = blockIdx.x; w < a.items; w += gridDim.x) {
        const uint32_t grp = fast_div(w, a.chunk_div);
        const uint32_t chunk = w - grp * a.chunks;
        const uint32_t g0 = grp * a.P;                // first position of the block
        const bool fill = t < a.entries && g0 + eq < a.bs;
        const uint32_t gq = min(g0 + eq, a.bs - 1);
        const uint32_t bq = fast_div(gq, a.s_div);
        const int64_t p0 = a.pos[(int64_t)bq * a.pos_sb + (int64_t)(gq - bq * a.s_div.d) * a.pos_ss];
        const double f0 = a.inv_freq[ei];
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t g = g0 + pp;
        const bool pos_live = g < a.bs;
        const uint32_t gl = pos_live ? g : a.bs - 1;  // past the last position: re-read it, store nothing
        const uint32_t n0 = chunk * (a.HL * U) + hl;
        v4u xa[U], xb[U];
        v4u* px[U];
        bool live[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t n = n0 + (uint32_t)k * a.HL;
            live[k] = pos_live && n < a.N;            // past N: re-read row N-1, store nothing
            const uint32_t nl = n < a.N ? n : a.N - 1;
            px[k] = pos_row_vec<MULTI>(a, gl, nl, cx);
            xa[k] = load_x<true>(px[k]);
            if constexpr (MODE == kModeRH) xb[k] = load_x<true>(px[k] + a.half_vecs);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (fill) cs[t] = pos_cos_sin<TT>(p0, f0);
        for (uint32_t e = t + blockDim.x; e < a.entries; e += blockDim.x) {
            const uint32_t q = fast_div(e, a.pairs_div);
            const uint32_t ge = g0 + q;
            if (ge >= a.bs) break;                    // later entries belong to later positions
            const uint32_t be = fast_div(ge, a.s_div);
            const int64_t pe = a.pos[(int64_t)be * a.pos_sb + (int64_t)(ge - be * a.s_div.d) * a.pos_ss];
            cs[e] = pos_cos_sin<TT>(pe, a.inv_freq[e - q * a.pairs]);
        }
        __syncthreads();
        // cos and sin of the thread's lanes: interleave lane j belongs to
        // pair j/2; rotate_half lane j of the first half to pair j, and the
        // matching lane of the second half shares it
        const uint32_t base = pp * a.pairs;
        float C[K], S[K];
#pragma unroll
        for (int e = 0; e < K; ++e) {
            const uint32_t i = MODE == kModeIL ? (v * K + e) / 2 : v * K + e;
            const float2 q = cs[in_slice && pos_live ? base + i : 0];
            C[e] = q.x;
            S[e] = q.y;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (!live[k] || !in_slice) continue;
            Lanes<DT> X;
            X.unpack(xa[k]);
            if constexpr (MODE == kModeIL) {
#pragma unroll
                for (int i = 0; i < K; i += 2)
                    rotate_pair<DIR, kUnfused>(X.v[i], X.v[i + 1], C[i], S[i], C[i + 1], S[i + 1]);
                store_x<true>(px[k], X.pack());
            } else {
                Lanes<DT> X2;
                X2.unpack(xb[k]);
#pragma unroll
                for (int i = 0; i < K; ++i) rotate_pair<DIR, kUnfused>(X.v[i], X2.v[i], C[i], S[i], C[i], S[i]);
                store_x<true>(px[k], X.pack());
                store_x<true>(px[k] + a.half_vecs, X2.pack());
            }
        }
        __syncthreads();   // the next item rewrites cs
    }
}

// Out of place with the tables computed from positions: x (the output)
// receives src with the slice rotated, in one pass over whole rows. A thread
// covers one vector of a row: outside the slice it copies it, inside it
// rotates it (interleave: the pairs within the vector; rotate_half: with the
// partner vector, the matching one in the other half of its group) and
// stores exactly that vector, with one instruction. XCHG: the partner vector
// comes from the lane that holds it (ds_bpermute; rows of 64/k vectors, so a
// row's threads never straddle a wave); otherwise it is loaded from src as
// well. Blocks, positions, loads and the LDS entries are those of the
// in-place kernel above.
template <int DT, int TT, int DIR, int MODE, bool XCHG>
__global__ void __launch_bounds__(256) rope_pos_out_kernel(PosArgs a)
{
    __shared__ float2 cs[kPosLds];
    constexpr int K = Store<DT>::kLanes;
    constexpr int U = pos_out_heads(MODE);
    constexpr bool kUnfused = DT != ROPE_DTYPE_F32;
    const uint32_t t = threadIdx.x;
    const uint32_t pp = fast_div(t, a.lanes_div);
    const uint32_t r = t - pp * a.lanes;
    const uint32_t hl = fast_div(r, a.span_div);
    const uint32_t c = r - hl * a.span;               // vector within the row (the threads cover the row)
    const uint32_t rel = c - a.start_vec;             // slice-relative (wraps below the slice)
    const bool in_slice = c >= a.start_vec && rel < (MODE == kModeIL ? a.nvec : 2 * a.nvec);
    // rotate_half: the group of the thread's vector, its place in the group,
    // whether it lies in the first half, its partner, and the first-half
    // unit whose lanes are pairs unit*K + e
    const uint32_t grp = MODE == kModeRH && in_slice ? rel / a.gvec : 0;
    const uint32_t grel = rel - grp * a.gvec;
    const bool first = MODE == kModeIL || grel < a.half_vecs;
    const uint32_t partner = MODE == kModeRH && in_slice ? (first ? c + a.half_vecs : c - a.half_vecs) : c;
    const uint32_t unit = grp * a.half_vecs + (first ? grel : grel - a.half_vecs);
    // the partner term is subtracted on the first half forward, on the second backward
    const bool neg = DIR == kFwd ? first : !first;
    // XCHG: byte address of the partner's lane for ds_bpermute (the lane
    // itself outside the slice)
    const int xlane = XCHG ? (int)((t & 63u) + (partner - c)) * 4 : 0;
    const uint32_t eq = fast_div(t, a.pairs_div);
    const uint32_t ei = t - eq * a.pairs;
    for (uint32_t w = blockIdx.x; w < a.items; w += gridDim.x) {
        const uint32_t grpb = fast_div(w, a.chunk_div);
        const uint32_t chunk = w - grpb * a.chunks;
        const uint32_t g0 = grpb * a.P;
        const bool fill = t < a.entries && g0 + eq < a.bs;
        const uint32_t gq = min(g0 + eq, a.bs - 1);
        const uint32_t bq = fast_div(gq, a.s_div);
        const int64_t p0 = a.pos[(int64_t)bq * a.pos_sb + (int64_t)(gq - bq * a.s_div.d) * a.pos_ss];
        const double f0 = a.inv_freq[ei];
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t g = g0 + pp;
        const bool pos_live = g < a.bs;
        const uint32_t gl = pos_live ? g : a.bs - 1;
        const uint32_t n0 = chunk * (a.HL * U) + hl;
        v4u xa[U], xb[U];
        uint32_t off[U];
        bool live[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t n = n0 + (uint32_t)k * a.HL;
            live[k] = pos_live && n < a.N;
            const uint32_t nl = n < a.N ? n : a.N - 1;
            const uint32_t row = (gl * a.N + nl) * a.row_vecs;
            off[k] = row + c;
            xa[k] = load_x<true>(a.src + off[k]);
            if constexpr (MODE == kModeRH && !XCHG) xb[k] = load_x<true>(a.src + row + partner);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE == kModeRH && XCHG) {
            // every lane takes part (no branch on the lane's own position yet)
#pragma unroll
            for (int k = 0; k < U; ++k) xb[k] = lane_exchange(xa[k], xlane);
        }
        if (fill) cs[t] = pos_cos_sin<TT>(p0, f0);
        for (uint32_t e = t + blockDim.x; e < a.entries; e += blockDim.x) {
            const uint32_t q = fast_div(e, a.pairs_div);
            const uint32_t ge = g0 + q;
            if (ge >= a.bs) break;
            const uint32_t be = fast_div(ge, a.s_div);
            const int64_t pe = a.pos[(int64_t)be * a.pos_sb + (int64_t)(ge - be * a.s_div.d) * a.pos_ss];
            cs[e] = pos_cos_sin<TT>(pe, a.inv_freq[e - q * a.pairs]);
        }
        __syncthreads();
        const uint32_t base = pp * a.pairs;
        float C[K], S[K];
#pragma unroll
        for (int e = 0; e < K; ++e) {
            const uint32_t i = MODE == kModeIL ? (rel * K + e) / 2 : unit * K + e;
            const float2 q = cs[in_slice && pos_live ? base + i : 0];
            C[e] = q.x;
            S[e] = q.y;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (!live[k]) continue;
            v4u y = xa[k];
            if (in_slice) {
                Lanes<DT> X;
                X.unpack(xa[k]);
                if constexpr (MODE == kModeIL) {
#pragma unroll
                    for (int i = 0; i < K; i += 2)
                        rotate_pair<DIR, kUnfused>(X.v[i], X.v[i + 1], C[i], S[i], C[i + 1], S[i + 1]);
                } else {
                    Lanes<DT> Pv;
                    Pv.unpack(xb[k]);
#pragma unroll
                    for (int i = 0; i < K; ++i) X.v[i] = rotate_own<kUnfused>(X.v[i], Pv.v[i], C[i], S[i], neg);
                }
                y = X.pack();
            }
            store_x<true>(a.x + off[k], y);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Scalar kernel: the general kernel from 2^31 rows on (the row kernel below
// takes fewer). Any alignment, any start parity, any slice length; one
// thread per rotation pair; 64-bit indexing throughout.
// ---------------------------------------------------------------------------
struct ScalarArgs {
    void* x;
    const void* r1;
    const void* r2;
    const int64_t* pos;     // POS: positions (position of (b,s) at pos[b*pos_sb + s*pos_ss])
    const double* inv_freq; // POS: L/2 frequencies
    int64_t pos_sb, pos_ss;
    int64_t S, N, D, start, L;
    int64_t half;           // rotate_half: lanes between a pair's lanes (L/2, or L/c for a coefficient c)
    int64_t pairs;          // pairs per row = L/2
    int64_t items;          // rows * pairs
    int64_t t1b, t1s, t1n;  // cos strides in elements (0 = broadcast)
    int64_t t2b, t2s, t2n;
};

template <int DT, int TT, int DIR, int MODE, bool POS>
__global__ void __launch_bounds__(256) rope_scalar_kernel(ScalarArgs a)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.items; i += stride) {
        const int64_t row = i / a.pairs;
        const int64_t q = i - row * a.pairs;
        // negated-partner lane: interleave 2q; rotate_half lane q % half of
        // the first half of group q / half (q itself when the slice is one group)
        const int64_t j = MODE == kModeIL ? 2 * q : (q / a.half) * 2 * a.half + q % a.half;
        const int64_t pj = MODE == kModeIL ? 2 * q + 1 : j + a.half;
        const int64_t n = row % a.N;
        const int64_t bs = row / a.N;
        const int64_t s = bs % a.S;
        const int64_t b = bs / a.S;
        const int64_t xo = row * a.D + a.start;
        float xa = Store<DT>::load1(a.x, xo + j);
        float xb = Store<DT>::load1(a.x, xo + pj);
        float ca, cb, sa, sb;
        if constexpr (POS) {
            // both lanes of pair q share its angle
            const float2 t = pos_cos_sin<TT>(a.pos[b * a.pos_sb + s * a.pos_ss], a.inv_freq[q]);
            ca = cb = t.x;
            sa = sb = t.y;
        } else {
            const int64_t co = b * a.t1b + s * a.t1s + n * a.t1n;
            const int64_t so = b * a.t2b + s * a.t2s + n * a.t2n;
            ca = Store<TT>::load1(a.r1, co + j);
            cb = Store<TT>::load1(a.r1, co + pj);
            sa = Store<TT>::load1(a.r2, so + j);
            sb = Store<TT>::load1(a.r2, so + pj);
        }
        rotate_pair<DIR, DT != ROPE_DTYPE_F32>(xa, xb, ca, sa, cb, sb);
        Store<DT>::store1(a.x, xo + j, xa);
        Store<DT>::store1(a.x, xo + pj, xb);
    }
}

// Row kernel: the general kernel for fewer than 2^31 rows. A block holds
// rpb rows of tpr threads; thread (lr, q0) of the block takes pairs q0,
// q0 + tpr, ... of row g*rpb + lr for each row group g it visits. The row,
// head and position come from launch-constant divisions (multiply-high and
// shift); element offsets stay 64-bit.
struct RowArgs {
    void* x;
    const void* r1;
    const void* r2;
    const int64_t* pos;     // POS: positions (position of (b,s) at pos[b*pos_sb + s*pos_ss])
    const double* inv_freq; // POS: L/2 frequencies
    int64_t pos_sb, pos_ss;
    int64_t D, start;       // row length and slice start, elements
    int64_t t1b, t1s, t1n;  // cos strides in elements (0 = broadcast)
    int64_t t2b, t2s, t2n;
    uint32_t L, pairs;      // slice length and rotation pairs per row
    uint32_t half;          // rotate_half: lanes between a pair's lanes (L/2, or L/c for a coefficient c)
    FastDiv half_div;
    uint32_t rows, N;
    uint32_t rpb, tpr;      // rows per block, threads per row
    uint32_t groups;        // ceil(rows / rpb)
    FastDiv tpr_div, n_div, s_div;
};

template <int DT, int TT, int DIR, int MODE, bool POS>
__global__ void __launch_bounds__(256) rope_rows_kernel(RowArgs a)
{
    const uint32_t t = threadIdx.x;
    const uint32_t lr = fast_div(t, a.tpr_div);
    const uint32_t q0 = t - lr * a.tpr;
    if (lr >= a.rpb) return;
    for (uint32_t g = blockIdx.x; g < a.groups; g += gridDim.x) {
        const uint32_t row = g * a.rpb + lr;
        if (row >= a.rows) return;  // later groups hold larger rows
        const uint32_t bs = fast_div(row, a.n_div);
        const uint32_t n = row - bs * a.N;
        const uint32_t b = fast_div(bs, a.s_div);
        const uint32_t s = bs - b * a.s_div.d;
        const int64_t xo = (int64_t)row * a.D + a.start;
        const int64_t co = b * a.t1b + s * a.t1s + n * a.t1n;
        const int64_t so = b * a.t2b + s * a.t2s + n * a.t2n;
        const int64_t p = POS ? a.pos[b * a.pos_sb + s * a.pos_ss] : 0;
        for (uint32_t q = q0; q < a.pairs; q += a.tpr) {
            // negated-partner lane (see the scalar kernel)
            const uint32_t g = MODE == kModeIL ? 0 : fast_div(q, a.half_div);
            const uint32_t j = MODE == kModeIL ? 2 * q : g * 2 * a.half + (q - g * a.half);
            const uint32_t pj = MODE == kModeIL ? 2 * q + 1 : j + a.half;
            float xa = Store<DT>::load1(a.x, xo + j);
            float xb = Store<DT>::load1(a.x, xo + pj);
            float ca, cb, sa, sb;
            if constexpr (POS) {
                // both lanes of pair q share its angle
                const float2 t = pos_cos_sin<TT>(p, a.inv_freq[q]);
                ca = cb = t.x;
                sa = sb = t.y;
            } else {
                ca = Store<TT>::load1(a.r1, co + j);
                cb = Store<TT>::load1(a.r1, co + pj);
                sa = Store<TT>::load1(a.r2, so + j);
                sb = Store<TT>::load1(a.r2, so + pj);
            }
            rotate_pair<DIR, DT != ROPE_DTYPE_F32>(xa, xb, ca, sa, cb, sb);
            Store<DT>::store1(a.x, xo + j, xa);
            Store<DT>::store1(a.x, xo + pj, xb);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
thread_local std::string g_last_error;

rope_status_t set_error(rope_status_t st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Heads per thread of the instantiated vector kernels: in place, and out of
// place (see prepare_out).
constexpr int kUInPlace = 1;
constexpr int kUOut = 2;

// Launch shape of the vector kernel.
struct VecConfig {
    int kmode = kModeIL;  // kernel scheme: kModeIL, kModeRH (pair owner) or kModeRHOwn
    int U = 1;          // heads per thread per tile (kUInPlace or kUOut)
    uint32_t HL = 1;    // head lanes per tile
    uint32_t GL = 1;    // tiles per block iteration
    uint32_t grid = 0;  // blocks; 0 = one block per tile group
    uint32_t xcd_group = 1;  // P of the XCD renumbering (1: dispatch order)
    bool nt = true;     // nontemporal loads/stores of x (the library instantiates true)
};

// Can the 16-byte vector kernel run this plan? Fills the geometry of `a`.
// Table types: the same as x, fp32 with 16-bit x, or 16-bit with fp32 x;
// fp16 with bf16 (either way round) takes the general kernel.
bool vec_geometry(const Plan& p, VecArgs* a)
{
    const int64_t es = p.esize, ts = p.tesize;
    if (p.tdtype != p.dtype && p.tdtype != ROPE_DTYPE_F32 && p.dtype != ROPE_DTYPE_F32) return false;
    const int64_t tbytes = 16 * ts / es;                   // table bytes per x vector: 8, 16 or 32
    const int64_t unit = std::min<int64_t>(16, tbytes);    // table unit (TableLanes::Vec)
    const int64_t tv = tbytes / unit;                      // table units per x vector: 1 or 2
    const auto aligned = [](const void* q, int64_t n) { return (reinterpret_cast<uintptr_t>(q) % n) == 0; };
    if (!aligned16(p.x) || !aligned(p.r1, unit) || !aligned(p.r2, unit)) return false;
    if ((p.D * es) % 16 || (p.start * es) % 16) return false;
    const int64_t unit_bytes = p.mode == kModeIL ? p.L * es : (p.L / 2) * es;
    if (unit_bytes % 16) return false;
    if (p.mode == kModeRH && (p.half * es) % 16) return false;   // half-groups of whole vectors
    for (int k = 0; k < 3; ++k)
        if ((p.t1[k] * ts) % unit || (p.t2[k] * ts) % unit) return false;
    // 32-bit offsets: x must span fewer than 2^32 vectors and each table
    // fewer than 2^32 units; tile indices stay below 2^31 (finish_vec_args).
    const int64_t kMax = (1ll << 32) - 1;
    const int64_t x_vecs = p.B * p.S * p.N * (p.D * es / 16);
    if (x_vecs > kMax || p.N >= (1ll << 31) || p.S >= (1ll << 31) || p.B * p.S >= (1ll << 31)) return false;
    const int64_t dims[3] = {p.B, p.S, p.N};
    int64_t t1_span = p.L * ts / unit, t2_span = p.L * ts / unit;
    for (int k = 0; k < 3; ++k) {
        t1_span += (dims[k] - 1) * (p.t1[k] * ts / unit);
        t2_span += (dims[k] - 1) * (p.t2[k] * ts / unit);
    }
    if (t1_span > kMax || t2_span > kMax) return false;
    a->x = static_cast<v4u*>(p.x);
    a->src = nullptr;
    a->r1 = p.r1;
    a->r2 = p.r2;
    a->row_vecs = (uint32_t)(p.D * es / 16);
    a->start_vec = (uint32_t)(p.start * es / 16);
    a->lo_vec = a->start_vec;
    a->half_vecs = p.mode == kModeRH ? (uint32_t)(p.half * es / 16) : 0;
    a->gvec = 2 * a->half_vecs;
    a->thalf = (uint32_t)(a->half_vecs * tv);
    a->t1b = (uint32_t)(p.t1[0] * ts / unit); a->t1s = (uint32_t)(p.t1[1] * ts / unit);
    a->t1n = (uint32_t)(p.t1[2] * ts / unit);
    a->t2b = (uint32_t)(p.t2[0] * ts / unit); a->t2s = (uint32_t)(p.t2[1] * ts / unit);
    a->t2n = (uint32_t)(p.t2[2] * ts / unit);
    a->N = (uint32_t)p.N;
    a->s_div = make_fastdiv((uint32_t)p.S);
    a->nvec = (uint32_t)(unit_bytes / 16);
    a->span = a->nvec;
    return a->nvec >= 1 && a->nvec <= 256;
}

// Slices that cover only part of their first or last 128-byte line
// (interleave, and rotate_half in the own-vector scheme): let the threads of
// a row cover the whole lines around the slice (see the vector kernel).
// Needs rows that start on line boundaries so the lines stay inside the row. Measured on MI355X for bf16 lanes [32,96) of
// 128 (same HBM bytes either way): 3-4% faster in this kernel, and 15% in a
// bare read-modify-write of the same bytes.
void cover_whole_lines(const Plan& p, VecArgs* a)
{
    const int64_t es = p.esize;
    const int64_t lo = (p.start * es) / 128 * 128;
    const int64_t hi = ((p.start + p.L) * es + 127) / 128 * 128;
    if (lo == p.start * es && hi == (p.start + p.L) * es) return;   // whole lines already
    if ((p.D * es) % 128 || (reinterpret_cast<uintptr_t>(p.x) & 127u)) return;
    if ((hi - lo) / 16 > 256) return;
    a->lo_vec = (uint32_t)(lo / 16);
    a->span = (uint32_t)((hi - lo) / 16);
}

// Launch shape for U heads per thread and a target block size: head lanes
// cover the heads of a (b,s) position up to the block size, and the rest of
// the block takes further tiles.
VecConfig shape_for(const VecArgs& a, int U, uint32_t threads)
{
    VecConfig c;
    c.U = U;
    const uint32_t hl_max = std::max<uint32_t>(1, threads / a.span);
    c.HL = (uint32_t)std::min<uint64_t>(hl_max, (a.N + U - 1) / U);
    c.GL = std::max<uint32_t>(1, threads / (a.span * c.HL));
    return c;
}

// The launch shape. Measured on MI355X with every launch reading data that
// no cache holds (the slices of several shapes: 1/4, 1/3, 1/2 and all of the
// row, whole and half 128-byte lines, bf16 and fp32, tables shared or per
// batch), sweeping heads per thread (1-8), block size (64-256) and
// nontemporal x: one head per thread, 64-thread blocks and nontemporal x was
// within 3% of the best shape on every one. Streaming x past the caches
// leaves the L2 to the tables, and small blocks let the dispatcher keep
// every CU's load queues full.
//
// XCD runs (see xcd_grouped_block): each XCD takes about kXcdRunBytes of
// consecutive rows of x per window, in whole (b,s) positions. Swept from one
// block to an eighth of the grid on twelve shapes: the time depends on the
// run length in a way that follows the HBM address interleave rather than
// the shape (runs of 16-64 KiB were 10-25% slower than the best), and runs
// of 384 KiB were within 4% of the best run length on all but the fp32
// shapes whose slice is a third of the row (there an eighth of the grid per
// XCD was 4% faster), and 7% faster than an eighth per XCD for the bf16
// long-context shard (16,8192,32,128) with lanes [32,96).
constexpr uint64_t kXcdRunBytes = 384u << 10;

VecConfig choose_vec_config(const Plan& p, const VecArgs& a, int U, int kmode)
{
    VecConfig c = shape_for(a, U, 64);
    c.kmode = kmode;
    c.nt = true;
    const uint64_t heads_per_tile = (uint64_t)c.HL * c.U;
    const uint64_t blocks_per_position = c.GL == 1 ? (a.N + heads_per_tile - 1) / heads_per_tile : 1;
    const uint64_t block_bytes = heads_per_tile * c.GL * (uint64_t)p.D * (uint64_t)p.esize;
    const uint64_t position_bytes = block_bytes * blocks_per_position;
    const uint64_t positions = std::max<uint64_t>(1, (kXcdRunBytes + position_bytes / 2) / position_bytes);
    c.xcd_group = (uint32_t)std::min<uint64_t>(positions * blocks_per_position, 1u << 24);
    return c;
}

// The dispatch packet holds the grid size in work-items as a 32-bit number.
constexpr uint64_t kMaxGridItems = 0xFFFFFFFFull;

uint32_t vec_grid(const VecArgs& a, const VecConfig& cfg)
{
    // One block per tile group by default: measured faster on MI355X than a
    // persistent grid for these streaming shapes (the dispatcher keeps every
    // CU full and no loop-carried dependence serialises the loads). A grid
    // that would exceed kMaxGridItems work-items is cut to fit, and the
    // blocks stride over the remaining tile groups.
    const uint64_t threads = (uint64_t)a.span * a.HL * a.GL;
    uint64_t grid = cfg.grid ? cfg.grid : a.btiles;
    grid = std::min<uint64_t>(grid, kMaxGridItems / threads);
    return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(grid, a.btiles));
}

// Complete `a` for a launch shape: head chunks and tile counts. False if a
// tile index could come near 32-bit wrap-around (the grid-stride loop adds
// gridDim.x to it), in which case a general kernel runs instead.
bool finish_vec_args(const Plan& p, const VecConfig& cfg, VecArgs* a)
{
    // The library instantiates the chosen shapes only: kUInPlace or kUOut
    // heads per thread, nontemporal x.
    if (cfg.U != (a->src ? kUOut : kUInPlace) || !cfg.nt || cfg.HL < 1 || cfg.GL < 1 ||
        (uint64_t)cfg.HL * cfg.GL * a->span > 256)
        return false;
    a->HL = cfg.HL;
    a->GL = cfg.GL;
    const uint64_t heads_per_tile = (uint64_t)cfg.HL * cfg.U;
    const uint64_t nchunk = (a->N + heads_per_tile - 1) / heads_per_tile;
    const uint64_t tiles = (uint64_t)p.B * p.S * nchunk;
    if (tiles >= (1ull << 31) || nchunk * heads_per_tile >= (1ull << 31)) return false;
    a->nchunk = (uint32_t)nchunk;
    a->tiles = (uint32_t)tiles;
    a->btiles = (uint32_t)((tiles + cfg.GL - 1) / cfg.GL);
    a->span_div = make_fastdiv(a->span);
    a->hl_div = make_fastdiv(a->HL);
    a->nchunk_div = make_fastdiv(a->nchunk);
    const uint64_t G = vec_grid(*a, cfg);
    const uint64_t P = std::max<uint32_t>(1, cfg.xcd_group);
    a->xcd_group = (uint32_t)P;
    a->xcd_full = 0;
    a->xcd_div = make_fastdiv(8);
    if (P > 1 && 8 * P <= G) {
        a->xcd_full = (uint32_t)(G / (8 * P) * (8 * P));
        a->xcd_div = make_fastdiv((uint32_t)(8 * P));
    }
    return true;
}

// Which vector kernel: in place on one tensor, in place on several, or out
// of place.
enum VecKind { kVecOne = 0, kVecMulti = 1, kVecOut = 2 };

template <int DT, int TT, int DIR, int MODE, bool SHARE>
const void* vec_kernel_ptr(VecKind kind)
{
    switch (kind) {
    case kVecMulti:
        // in place: no memory partner loads
        if constexpr (MODE == kModeRHOwnLoad) return nullptr;
        else return reinterpret_cast<const void*>(&rope_vec_multi_kernel<DT, TT, DIR, MODE, kUInPlace, SHARE, true>);
    case kVecOut:
        // out of place, rotate_half always takes an own-vector scheme
        if constexpr (MODE == kModeRH) return nullptr;
        else return reinterpret_cast<const void*>(&rope_vec_out_kernel<DT, TT, DIR, MODE, kUOut, SHARE, true>);
    default:
        if constexpr (MODE == kModeRHOwnLoad) return nullptr;
        else return reinterpret_cast<const void*>(&rope_vec_kernel<DT, TT, DIR, MODE, kUInPlace, SHARE, true>);
    }
}

template <int DT, int TT, int DIR, int MODE>
const void* vec_kernel_s(bool share, VecKind kind)
{
    return share ? vec_kernel_ptr<DT, TT, DIR, MODE, true>(kind) : vec_kernel_ptr<DT, TT, DIR, MODE, false>(kind);
}

template <int DT, int TT, int DIR>
const void* vec_kernel_m(int kmode, bool share, VecKind kind)
{
    switch (kmode) {
    case kModeIL: return vec_kernel_s<DT, TT, DIR, kModeIL>(share, kind);
    case kModeRH: return vec_kernel_s<DT, TT, DIR, kModeRH>(share, kind);
    case kModeRHOwn: return vec_kernel_s<DT, TT, DIR, kModeRHOwn>(share, kind);
    default: return vec_kernel_s<DT, TT, DIR, kModeRHOwnLoad>(share, kind);
    }
}

template <int DT, int TT>
const void* vec_kernel_t(int dir, int kmode, bool share, VecKind kind)
{
    return dir == kFwd ? vec_kernel_m<DT, TT, kFwd>(kmode, share, kind) : vec_kernel_m<DT, TT, kBwd>(kmode, share, kind);
}

// The vector kernel instance for a plan that vec_geometry accepted, in the
// scheme `kmode` (VecConfig::kmode).
const void* vec_kernel(const Plan& p, int kmode, VecKind kind)
{
    const bool share = p.t1[2] == 0 && p.t2[2] == 0;
    const int tt = p.tdtype;
    switch (p.dtype) {
    case ROPE_DTYPE_F32:
        if (tt == ROPE_DTYPE_F16) return vec_kernel_t<ROPE_DTYPE_F32, ROPE_DTYPE_F16>(p.dir, kmode, share, kind);
        if (tt == ROPE_DTYPE_BF16) return vec_kernel_t<ROPE_DTYPE_F32, ROPE_DTYPE_BF16>(p.dir, kmode, share, kind);
        return vec_kernel_t<ROPE_DTYPE_F32, ROPE_DTYPE_F32>(p.dir, kmode, share, kind);
    case ROPE_DTYPE_F16:
        return tt == ROPE_DTYPE_F32 ? vec_kernel_t<ROPE_DTYPE_F16, ROPE_DTYPE_F32>(p.dir, kmode, share, kind)
                                    : vec_kernel_t<ROPE_DTYPE_F16, ROPE_DTYPE_F16>(p.dir, kmode, share, kind);
    default:
        return tt == ROPE_DTYPE_F32 ? vec_kernel_t<ROPE_DTYPE_BF16, ROPE_DTYPE_F32>(p.dir, kmode, share, kind)
                                    : vec_kernel_t<ROPE_DTYPE_BF16, ROPE_DTYPE_BF16>(p.dir, kmode, share, kind);
    }
}

// Launch the vector kernel; `a` is complete (vec_geometry + finish_vec_args).
// a.src set means out of place.
hipError_t launch_vec(const Plan& p, const VecArgs& a, const VecConfig& cfg, hipStream_t stream)
{
    const uint32_t threads = a.span * a.HL * a.GL;
    const void* fn = vec_kernel(p, cfg.kmode, a.src ? kVecOut : kVecOne);
    if (fn == nullptr) return hipErrorInvalidDeviceFunction;
    void* args[] = {const_cast<VecArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(vec_grid(a, cfg)), dim3(threads), args, 0, stream);
}

template <int DT, int TT, bool POS>
const void* scalar_kernel_t(int dir, int mode)
{
    if (dir == kFwd)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kFwd, kModeIL, POS>)
                               : reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kFwd, kModeRH, POS>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kBwd, kModeIL, POS>)
                           : reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kBwd, kModeRH, POS>);
}

template <int DT, int TT>
const void* scalar_kernel_p(bool pos, int dir, int mode)
{
    return pos ? scalar_kernel_t<DT, TT, true>(dir, mode) : scalar_kernel_t<DT, TT, false>(dir, mode);
}

template <int DT>
const void* scalar_kernel_dt(int tt, bool pos, int dir, int mode)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return scalar_kernel_p<DT, ROPE_DTYPE_F32>(pos, dir, mode);
    case ROPE_DTYPE_F16: return scalar_kernel_p<DT, ROPE_DTYPE_F16>(pos, dir, mode);
    default: return scalar_kernel_p<DT, ROPE_DTYPE_BF16>(pos, dir, mode);
    }
}

hipError_t launch_scalar(const Plan& p, int cus, hipStream_t stream)
{
    ScalarArgs a;
    a.x = p.x; a.r1 = p.r1; a.r2 = p.r2;
    a.pos = p.pos; a.inv_freq = p.inv_freq; a.pos_sb = p.pos_sb; a.pos_ss = p.pos_ss;
    a.S = p.S; a.N = p.N; a.D = p.D; a.start = p.start; a.L = p.L;
    a.half = p.half;
    a.pairs = p.L / 2;
    a.items = p.B * p.S * p.N * a.pairs;
    a.t1b = p.t1[0]; a.t1s = p.t1[1]; a.t1n = p.t1[2];
    a.t2b = p.t2[0]; a.t2s = p.t2[1]; a.t2n = p.t2[2];
    const uint32_t threads = 256;
    uint64_t grid = (uint64_t)cus * 8;
    grid = std::max<uint64_t>(1, std::min<uint64_t>(grid, (a.items + threads - 1) / threads));
    const void* fn;
    switch (p.dtype) {
    case ROPE_DTYPE_F32: fn = scalar_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    case ROPE_DTYPE_F16: fn = scalar_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    default: fn = scalar_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(threads), args, 0, stream);
}

template <int DT, int TT, bool POS>
const void* rows_kernel_t(int dir, int mode)
{
    if (dir == kFwd)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kFwd, kModeIL, POS>)
                               : reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kFwd, kModeRH, POS>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kBwd, kModeIL, POS>)
                           : reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kBwd, kModeRH, POS>);
}

template <int DT, int TT>
const void* rows_kernel_p(bool pos, int dir, int mode)
{
    return pos ? rows_kernel_t<DT, TT, true>(dir, mode) : rows_kernel_t<DT, TT, false>(dir, mode);
}

template <int DT>
const void* rows_kernel_dt(int tt, bool pos, int dir, int mode)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return rows_kernel_p<DT, ROPE_DTYPE_F32>(pos, dir, mode);
    case ROPE_DTYPE_F16: return rows_kernel_p<DT, ROPE_DTYPE_F16>(pos, dir, mode);
    default: return rows_kernel_p<DT, ROPE_DTYPE_BF16>(pos, dir, mode);
    }
}

// Launch shape of the row kernel: up to 256 threads per row (longer rows
// loop), as many whole rows per block as fit in 256 threads, one block per
// row group while the grid fits the dispatch packet.
struct RowShape {
    uint32_t tpr = 1, rpb = 1, threads = 1, groups = 0, grid = 0;
};

bool rows_shape(const Plan& p, RowShape* r)
{
    const uint64_t rows = (uint64_t)p.B * p.S * p.N;
    if (rows >= (1ull << 31)) return false;
    const uint32_t pairs = (uint32_t)(p.L / 2);
    r->tpr = std::min<uint32_t>(pairs, 256);
    r->rpb = 256 / r->tpr;
    r->threads = r->tpr * r->rpb;
    r->groups = (uint32_t)((rows + r->rpb - 1) / r->rpb);
    r->grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(r->groups, kMaxGridItems / r->threads));
    return true;
}

hipError_t launch_rows(const Plan& p, const RowShape& r, hipStream_t stream)
{
    RowArgs a;
    a.x = p.x; a.r1 = p.r1; a.r2 = p.r2;
    a.pos = p.pos; a.inv_freq = p.inv_freq; a.pos_sb = p.pos_sb; a.pos_ss = p.pos_ss;
    a.D = p.D; a.start = p.start;
    a.t1b = p.t1[0]; a.t1s = p.t1[1]; a.t1n = p.t1[2];
    a.t2b = p.t2[0]; a.t2s = p.t2[1]; a.t2n = p.t2[2];
    a.L = (uint32_t)p.L;
    a.pairs = (uint32_t)(p.L / 2);
    a.half = (uint32_t)std::max<int64_t>(1, p.half);
    a.half_div = make_fastdiv(a.half);
    a.rows = (uint32_t)(p.B * p.S * p.N);
    a.N = (uint32_t)p.N;
    a.rpb = r.rpb;
    a.tpr = r.tpr;
    a.groups = r.groups;
    a.tpr_div = make_fastdiv(r.tpr);
    a.n_div = make_fastdiv((uint32_t)p.N);
    a.s_div = make_fastdiv((uint32_t)p.S);
    const void* fn;
    switch (p.dtype) {
    case ROPE_DTYPE_F32: fn = rows_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    case ROPE_DTYPE_F16: fn = rows_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    default: fn = rows_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3(r.grid), dim3(r.threads), args, 0, stream);
}

// One tensor's launch, decided on the host.
struct Launch {
    Plan p;
    bool vec = false;
    VecArgs a{};
    VecConfig cfg;
    bool rows = false;  // row kernel (else the 64-bit scalar kernel) when not vec
    RowShape rs;
};

// In place, rotate_half: the pair-owner scheme requests each half with its
// own wave instruction, which covers whole 128-byte lines only when the
// halves start and end on line boundaries (e.g. a whole bf16 head of 128
// lanes). Otherwise take the own-vector scheme, whose threads cover the
// slice's whole lines -- when a row's threads fit one wave, as that scheme
// needs. Measured on MI355X, (16,4096,32,128) bf16 forward: lanes [64,128)
// 113 -> 86 us (the interleave slice of the same bytes takes 85 us), lanes
// [0,32) 95 -> 74 us. With the partner loaded from memory instead of taken
// from its lane, each line was requested twice: 100 and 76 us.
bool use_rh_own(const Plan& p, VecArgs* a)
{
    const int64_t es = p.esize;
    const int64_t half_bytes = p.half * es;
    if ((p.start * es) % 128 == 0 && half_bytes % 128 == 0) return false;   // halves on whole lines
    VecArgs own = *a;
    own.span = 2 * own.nvec;   // the whole slice
    cover_whole_lines(p, &own);
    if (own.span > 64) {       // the whole lines would not fit one wave: the slice alone may
        own.lo_vec = own.start_vec;
        own.span = 2 * own.nvec;
    }
    if (own.span > 64) return false;   // a row's threads would span waves
    *a = own;
    return true;
}

void prepare(Launch* L)
{
    L->vec = vec_geometry(L->p, &L->a);
    if (L->vec) {
        int kmode = L->p.mode;
        if (L->p.mode == kModeRH) {
            if (use_rh_own(L->p, &L->a)) kmode = kModeRHOwn;
        } else {
            cover_whole_lines(L->p, &L->a);
        }
        L->cfg = choose_vec_config(L->p, L->a, kUInPlace, kmode);
        L->vec = finish_vec_args(L->p, L->cfg, &L->a);
        // the own-vector scheme in place needs single-wave blocks
        if (L->vec && kmode == kModeRHOwn && L->a.span * L->a.HL * L->a.GL > 64) L->vec = false;
    }
    if (!L->vec) L->rows = rows_shape(L->p, &L->rs);
}

hipError_t launch_one(const Launch& L, int cus, hipStream_t s)
{
    if (L.vec) return launch_vec(L.p, L.a, L.cfg, s);
    return L.rows ? launch_rows(L.p, L.rs, s) : launch_scalar(L.p, cus, s);
}

// Out of place (p.src is the input, p.x the output; distinct buffers). The
// vector kernel reads src and writes x in one pass over whole rows: the
// slice rotated, the other vectors copied. Inputs it cannot take (alignment,
// sizes) get a device copy of src into x and then the in-place plan on x.
//
// Launch shape, measured on MI355X over six shapes (bf16 and fp32; slices
// of 1/3, 1/2 and all of the row; interleave and rotate_half; slices on and
// off 128-byte line boundaries), heads per thread 1-2, blocks of 64-256
// threads, and plain or nontemporal loads and stores chosen separately: two
// heads per thread, 64-thread blocks and nontemporal loads and stores was
// within 2% of the best on five shapes and 8% on the sixth (a rotate_half
// slice off line boundaries). One head per thread was 10-15% slower on the
// rotate_half shapes and the 192-lane rows. With every vector stored by one
// instruction (see the vector kernel) the long-context shard (16,8192,32,128)
// bf16 takes 322 us, 6.8 TB/s of read plus write, against 420 us for a
// plain device copy of the same tensor.
void prepare_out(Launch* L)
{
    L->vec = vec_geometry(L->p, &L->a) && aligned16(L->p.src);
    if (L->vec) {
        L->a.src = static_cast<const v4u*>(L->p.src);
        L->a.lo_vec = 0;
        L->a.span = L->a.row_vecs;
        // rotate_half: the partner vector from its lane when a row fits a wave
        const int kmode = L->p.mode == kModeIL ? kModeIL : L->a.span <= 64 ? kModeRHOwn : kModeRHOwnLoad;
        L->cfg = choose_vec_config(L->p, L->a, kUOut, kmode);
        L->vec = finish_vec_args(L->p, L->cfg, &L->a);
        // the lane exchange needs single-wave blocks
        if (L->vec && kmode == kModeRHOwn && L->a.span * L->a.HL * L->a.GL > 64) L->vec = false;
    }
    if (!L->vec) L->rows = rows_shape(L->p, &L->rs);
}

hipError_t launch_out(const Launch& L, int cus, hipStream_t s)
{
    if (L.vec) return launch_vec(L.p, L.a, L.cfg, s);
    hipError_t err = hipMemcpyAsync(L.p.x, L.p.src, (size_t)L.p.bytes, hipMemcpyDeviceToDevice, s);
    if (err != hipSuccess) return err;
    return L.rows ? launch_rows(L.p, L.rs, s) : launch_scalar(L.p, cus, s);
}

rope_status_t device_cus(int* cus)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("hipGetDevice: ") + hipGetErrorString(err));
    *cus = cu_count(dev);
    return ROPE_OK;
}

rope_status_t run(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                  const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                  const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                  rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                  void* stream, Direction dir)
{
    Launch L;
    std::string why;
    rope_status_t st = make_plan(x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                                 table_dtype, mode, partial_slice, dir, &L.p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (L.p.noop) return ROPE_OK;
    int cus = 0;
    if ((st = device_cus(&cus)) != ROPE_OK) return st;
    prepare(&L);
    hipError_t err = launch_one(L, cus, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Launch plan of the position vector kernel; false if the plan needs a
// general kernel (alignment, sizes), as for the table vector kernel. A
// position's heads take up to kPosLanes threads (HL head lanes of span
// threads, kUPos heads each, in chunks past kUPos*HL heads); when they fill
// fewer threads, a block takes kPosLanes/lanes positions, as many as its
// LDS table holds.
// The vector geometry both position kernels share: alignment, sizes, the
// slice in vectors and the rotate_half groups. out: also src aligned.
static bool pos_vectors(const Plan& p, PosArgs* a, bool out)
{
    const int64_t es = p.esize;
    if (!aligned16(p.x) || (out && !aligned16(p.src)) || (p.D * es) % 16 || (p.start * es) % 16) return false;
    const int64_t unit_bytes = p.mode == kModeIL ? p.L * es : (p.L / 2) * es;
    if (unit_bytes % 16 || p.L / 2 > kPosLds) return false;
    if (p.mode == kModeRH && (p.half * es) % 16) return false;   // half-groups of whole vectors
    const int64_t kMax = (1ll << 32) - 1;
    if (p.B * p.S * p.N * (p.D * es / 16) > kMax || p.N >= (1ll << 31) || p.B * p.S >= (1ll << 31)) return false;
    a->x = static_cast<v4u*>(p.x);
    a->src = static_cast<const v4u*>(p.src);
    a->pos = p.pos;
    a->inv_freq = p.inv_freq;
    a->pos_sb = p.pos_sb;
    a->pos_ss = p.pos_ss;
    a->row_vecs = (uint32_t)(p.D * es / 16);
    a->start_vec = (uint32_t)(p.start * es / 16);
    a->half_vecs = p.mode == kModeRH ? (uint32_t)(p.half * es / 16) : 0;
    a->gvec = 2 * a->half_vecs;
    a->nvec = (uint32_t)(unit_bytes / 16);
    return true;
}

// Heads, positions per block and the grid, once the vectors a row's
// threads cover (lo_vec, span) are set: U heads per thread, a position's
// heads over up to `lanes_target` threads.
static bool pos_launch_shape(const Plan& p, PosArgs* a, uint32_t* threads, uint32_t* grid, int U,
                             uint32_t lanes_target)
{
    if (a->span < 1 || a->span > 256) return false;
    a->N = (uint32_t)p.N;
    a->pairs = (uint32_t)(p.L / 2);
    a->HL = (uint32_t)std::min<uint64_t>(std::max<uint32_t>(1, lanes_target / a->span), (uint64_t)p.N);
    a->chunks = (uint32_t)((p.N + (uint64_t)a->HL * U - 1) / ((uint64_t)a->HL * U));
    a->lanes = a->span * a->HL;
    a->P = a->lanes < lanes_target ? std::min<uint32_t>(lanes_target / a->lanes, kPosLds / a->pairs) : 1;
    a->entries = a->P * a->pairs;
    if (a->entries > (uint32_t)kPosLds) return false;
    a->bs = (uint32_t)(p.B * p.S);
    const uint64_t items = (((uint64_t)a->bs + a->P - 1) / a->P) * a->chunks;
    if (items >= (1ull << 31)) return false;
    a->items = (uint32_t)items;
    *threads = a->P * a->lanes;
    *grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(items, kMaxGridItems / *threads));
    a->span_div = make_fastdiv(a->span);
    a->lanes_div = make_fastdiv(a->lanes);
    a->pairs_div = make_fastdiv(a->pairs);
    a->chunk_div = make_fastdiv(a->chunks);
    a->s_div = make_fastdiv((uint32_t)p.S);
    return true;
}

bool pos_geometry(const Plan& p, PosArgs* a, uint32_t* threads, uint32_t* grid)
{
    if (!pos_vectors(p, a, false)) return false;
    a->lo_vec = a->start_vec;
    a->span = a->nvec;
    if (p.mode == kModeIL) {
        VecArgs lines{};
        lines.lo_vec = a->lo_vec;
        lines.span = a->span;
        cover_whole_lines(p, &lines);
        a->lo_vec = lines.lo_vec;
        a->span = lines.span;
    }
    return pos_launch_shape(p, a, threads, grid, kUPos, kPosLanes);
}

// Out of place: the threads of a row cover all of its vectors.
bool pos_geometry_out(const Plan& p, PosArgs* a, uint32_t* threads, uint32_t* grid)
{
    if (!pos_vectors(p, a, true)) return false;
    a->lo_vec = 0;
    a->span = a->row_vecs;
    return pos_launch_shape(p, a, threads, grid, pos_out_heads(p.mode), pos_out_lanes(p.mode));
}

template <int DT, int TT, int DIR>
const void* pos_kernel_d(int mode, bool out, bool xchg)
{
    if (out)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_out_kernel<DT, TT, DIR, kModeIL, false>)
               : xchg          ? reinterpret_cast<const void*>(&rope_pos_out_kernel<DT, TT, DIR, kModeRH, true>)
                               : reinterpret_cast<const void*>(&rope_pos_out_kernel<DT, TT, DIR, kModeRH, false>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeIL, false>)
                           : reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeRH, false>);
}

template <int DT, int TT, int DIR>
const void* pos_multi_kernel_d(int mode)
{
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeIL, true>)
                           : reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeRH, true>);
}

template <int DT, int TT>
const void* pos_multi_kernel_t(int dir, int mode)
{
    return dir == kFwd ? pos_multi_kernel_d<DT, TT, kFwd>(mode) : pos_multi_kernel_d<DT, TT, kBwd>(mode);
}

template <int DT>
const void* pos_multi_kernel_dt(int tt, int dir, int mode)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return pos_multi_kernel_t<DT, ROPE_DTYPE_F32>(dir, mode);
    case ROPE_DTYPE_F16: return pos_multi_kernel_t<DT, ROPE_DTYPE_F16>(dir, mode);
    default: return pos_multi_kernel_t<DT, ROPE_DTYPE_BF16>(dir, mode);
    }
}

// the position kernel over several tensors at once
const void* pos_multi_kernel(const Plan& p)
{
    switch (p.dtype) {
    case ROPE_DTYPE_F32: return pos_multi_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.dir, p.mode);
    case ROPE_DTYPE_F16: return pos_multi_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.dir, p.mode);
    default: return pos_multi_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.dir, p.mode);
    }
}

template <int DT, int TT>
const void* pos_kernel_t(int dir, int mode, bool out, bool xchg)
{
    return dir == kFwd ? pos_kernel_d<DT, TT, kFwd>(mode, out, xchg) : pos_kernel_d<DT, TT, kBwd>(mode, out, xchg);
}

template <int DT>
const void* pos_kernel_dt(int tt, int dir, int mode, bool out, bool xchg)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return pos_kernel_t<DT, ROPE_DTYPE_F32>(dir, mode, out, xchg);
    case ROPE_DTYPE_F16: return pos_kernel_t<DT, ROPE_DTYPE_F16>(dir, mode, out, xchg);
    default: return pos_kernel_t<DT, ROPE_DTYPE_BF16>(dir, mode, out, xchg);
    }
}

// out: the out-of-place kernel; xchg: its lane exchange (a row's threads
// within one wave: rows of 64/k vectors)
const void* pos_kernel(const Plan& p, bool out, bool xchg = false)
{
    switch (p.dtype) {
    case ROPE_DTYPE_F32: return pos_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.dir, p.mode, out, xchg);
    case ROPE_DTYPE_F16: return pos_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.dir, p.mode, out, xchg);
    default: return pos_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.dir, p.mode, out, xchg);
    }
}

// Tables from positions, one planned tensor: the position vector kernel,
// else the row or scalar kernel with their POS form.
hipError_t launch_pos_plan(const Plan& p, int cus, hipStream_t s)
{
    PosArgs a{};
    uint32_t threads = 0, grid = 0;
    if (pos_geometry(p, &a, &threads, &grid)) {
        void* args[] = {&a};
        return hipLaunchKernel(pos_kernel(p, false), dim3(grid), dim3(threads), args, 0, s);
    }
    RowShape rs;
    return rows_shape(p, &rs) ? launch_rows(p, rs, s) : launch_scalar(p, cus, s);
}

rope_status_t run_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype, const int64_t* positions,
                      const int64_t positions_shape[2], const int64_t positions_strides[2], const double* inv_freq,
                      rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2], void* stream,
                      Direction dir)
{
    Plan p;
    std::string why;
    rope_status_t st = make_plan_pos(x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq,
                                     table_dtype, mode, partial_slice, dir, &p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (p.noop) return ROPE_OK;
    int cus = 0;
    if ((st = device_cus(&cus)) != ROPE_OK) return st;
    const hipError_t err = launch_pos_plan(p, cus, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Several tensors with one set of positions (the Q and K of a layer): every
// tensor is checked first; when they share B, S, D and the vector geometry,
// one launch of the position kernel takes the heads of all of them, each
// pair's cos and sin evaluated once per position for every tensor;
// otherwise one launch per tensor.
rope_status_t run_pos_multi(int32_t count, void* const xs[], const int64_t (*x_shapes)[4], rope_dtype_t dtype,
                            const int64_t* positions, const int64_t positions_shape[2],
                            const int64_t positions_strides[2], const double* inv_freq, rope_dtype_t table_dtype,
                            int64_t mode, const int64_t partial_slice[2], void* stream, Direction dir)
{
    if (count < 0 || count > kMultiMax)
        return set_error(ROPE_ERR_INVALID, "count must be in [0, " + std::to_string(kMultiMax) + "]");
    if (count == 0) return ROPE_OK;
    if (xs == nullptr || x_shapes == nullptr) return set_error(ROPE_ERR_NULLPTR, "xs or x_shapes is NULL");
    Plan P[kMultiMax];
    int live = 0;
    for (int i = 0; i < count; ++i) {
        std::string why;
        rope_status_t st = make_plan_pos(xs[i], x_shapes[i], dtype, positions, positions_shape, positions_strides,
                                         inv_freq, table_dtype, mode, partial_slice, dir, &P[live], &why);
        if (st != ROPE_OK) return set_error(st, "tensor " + std::to_string(i) + ": " + why);
        if (!P[live].noop) ++live;
    }
    if (live == 0) return ROPE_OK;
    int cus = 0;
    rope_status_t st = device_cus(&cus);
    if (st != ROPE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool together = live > 1;
    PosArgs each[kMultiMax];
    uint64_t heads = 0;
    for (int i = 0; i < live && together; ++i) {
        uint32_t t = 0, g = 0;
        together = P[i].B == P[0].B && P[i].S == P[0].S && P[i].D == P[0].D &&
                   pos_geometry(P[i], &each[i], &t, &g) && each[i].lo_vec == each[0].lo_vec &&
                   each[i].span == each[0].span;
        heads += (uint64_t)P[i].N;
    }
    hipError_t err = hipSuccess;
    PosArgs m{};
    uint32_t threads = 0, grid = 0;
    if (together && heads < (1ull << 31)) {
        Plan q = P[0];
        q.N = (int64_t)heads;
        m = each[0];
        together = pos_launch_shape(q, &m, &threads, &grid, kUPos, kPosLanes);
        uint32_t first = 0;
        for (int i = 0; i < kMultiMax; ++i) {
            m.xs[i] = i < live ? each[i].x : nullptr;
            m.nt[i] = i < live ? (uint32_t)P[i].N : 0;
            m.hoff[i] = i < live ? first : 0xFFFFFFFFu;
            if (i < live) first += (uint32_t)P[i].N;
        }
    } else {
        together = false;
    }
    if (together) {
        void* args[] = {&m};
        err = hipLaunchKernel(pos_multi_kernel(P[0]), dim3(grid), dim3(threads), args, 0, s);
    } else {
        for (int i = 0; i < live && err == hipSuccess; ++i) err = launch_pos_plan(P[i], cus, s);
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Out of place from positions: the position out-of-place kernel, else a
// device copy of x into y and the in-place position plan on y.
rope_status_t run_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                          const int64_t* positions, const int64_t positions_shape[2],
                          const int64_t positions_strides[2], const double* inv_freq, rope_dtype_t table_dtype,
                          int64_t mode, const int64_t partial_slice[2], void* stream, Direction dir)
{
    Plan p;
    std::string why;
    rope_status_t st = make_plan_out_pos(y, x, x_shape, dtype, positions, positions_shape, positions_strides,
                                         inv_freq, table_dtype, mode, partial_slice, dir, &p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (p.noop) return ROPE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (p.copy_only) {
        err = hipMemcpyAsync(p.x, p.src, (size_t)p.bytes, hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("copy: ") + hipGetErrorString(err));
        return ROPE_OK;
    }
    if (p.src == nullptr)   // y == x: the in-place call
        return run_pos(p.x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq, table_dtype,
                       mode, partial_slice, stream, dir);
    int cus = 0;
    if ((st = device_cus(&cus)) != ROPE_OK) return st;
    PosArgs a{};
    uint32_t threads = 0, grid = 0;
    if (pos_geometry_out(p, &a, &threads, &grid)) {
        void* args[] = {&a};
        const bool xchg = a.span <= 64 && 64 % a.span == 0;
        err = hipLaunchKernel(pos_kernel(p, true, xchg), dim3(grid), dim3(threads), args, 0, s);
    } else {
        err = hipMemcpyAsync(p.x, p.src, (size_t)p.bytes, hipMemcpyDeviceToDevice, s);
        if (err == hipSuccess) err = launch_pos_plan(p, cus, s);
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Out of place: y = x with the slice rotated (y == x is the in-place call).
rope_status_t run_out(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                      const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                      const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                      rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                      void* stream, Direction dir)
{
    Launch L;
    std::string why;
    rope_status_t st = make_plan_out(y, x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                                     table_dtype, mode, partial_slice, dir, &L.p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (L.p.noop) return ROPE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (L.p.copy_only) {
        err = hipMemcpyAsync(L.p.x, L.p.src, (size_t)L.p.bytes, hipMemcpyDeviceToDevice, s);
    } else {
        int cus = 0;
        if ((st = device_cus(&cus)) != ROPE_OK) return st;
        if (L.p.src == nullptr) {
            prepare(&L);
            err = launch_one(L, cus, s);
        } else {
            prepare_out(&L);
            err = launch_out(L, cus, s);
        }
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Several tensors with shared tables: every tensor is checked before any
// launch; tensors that all take the same vector kernel and block size go in
// one launch, otherwise each is launched in turn (same result either way).
rope_status_t run_multi(int32_t count, void* const xs[], const int64_t (*x_shapes)[4], rope_dtype_t dtype,
                        const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                        const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                        rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                        void* stream, Direction dir)
{
    if (count < 0 || count > kMultiMax)
        return set_error(ROPE_ERR_INVALID, "count must be in [0, " + std::to_string(kMultiMax) + "]");
    if (count == 0) return ROPE_OK;
    if (xs == nullptr || x_shapes == nullptr) return set_error(ROPE_ERR_NULLPTR, "xs or x_shapes is NULL");
    Launch L[kMultiMax];
    int live = 0;
    for (int i = 0; i < count; ++i) {
        std::string why;
        rope_status_t st = make_plan(xs[i], x_shapes[i], dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                                     table_dtype, mode, partial_slice, dir, &L[live].p, &why);
        if (st != ROPE_OK) return set_error(st, "tensor " + std::to_string(i) + ": " + why);
        if (!L[live].p.noop) ++live;
    }
    if (live == 0) return ROPE_OK;
    int cus = 0;
    rope_status_t st = device_cus(&cus);
    if (st != ROPE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i = 0; i < live; ++i) prepare(&L[i]);

    bool together = live > 1;
    const uint32_t threads = L[0].a.span * L[0].a.HL * L[0].a.GL;
    const void* fn = together && L[0].vec ? vec_kernel(L[0].p, L[0].cfg.kmode, kVecMulti) : nullptr;
    for (int i = 0; i < live && together; ++i) {
        together = L[i].vec && L[i].a.span * L[i].a.HL * L[i].a.GL == threads &&
                   vec_kernel(L[i].p, L[i].cfg.kmode, kVecMulti) == fn && L[i].cfg.grid == 0;
    }
    hipError_t err = hipSuccess;
    if (together) {
        MultiVecArgs m{};
        m.count = (uint32_t)live;
        uint64_t blocks = 0;
        for (int i = 0; i < live; ++i) {
            m.a[i] = L[i].a;
            m.first_block[i] = (uint32_t)blocks;
            blocks += vec_grid(L[i].a, L[i].cfg);
        }
        for (int i = live; i <= kMultiMax; ++i) m.first_block[i] = (uint32_t)blocks;
        if (blocks * threads > kMaxGridItems) together = false;
        if (together) {
            void* args[] = {&m};
            err = hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(threads), args, 0, s);
        }
    }
    if (!together) {
        for (int i = 0; i < live && err == hipSuccess; ++i) err = launch_one(L[i], cus, s);
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

}  // namespace
}  // namespace rope

extern "C" {

rope_status_t rope_partial_fwd_inplace(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run(x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype, mode,
                     partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run(x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype, mode,
                     partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_out(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                   const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                   const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                   rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                   void* stream)
{
    return rope::run_out(y, x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype,
                         mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_out(void* dx, const void* dy, const int64_t x_shape[4], rope_dtype_t dtype,
                                   const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                   const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                   rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                   void* stream)
{
    return rope::run_out(dx, dy, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype,
                         mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_inplace_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                           const int64_t* positions, const int64_t positions_shape[2],
                                           const int64_t positions_strides[2], const double* inv_freq,
                                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                           void* stream)
{
    return rope::run_pos(x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq, table_dtype,
                         mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                           const int64_t* positions, const int64_t positions_shape[2],
                                           const int64_t positions_strides[2], const double* inv_freq,
                                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                           void* stream)
{
    return rope::run_pos(x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq, table_dtype,
                         mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_inplace_pos_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                                 rope_dtype_t dtype, const int64_t* positions,
                                                 const int64_t positions_shape[2], const int64_t positions_strides[2],
                                                 const double* inv_freq, rope_dtype_t table_dtype, int64_t mode,
                                                 const int64_t partial_slice[2], void* stream)
{
    return rope::run_pos_multi(count, xs, x_shapes, dtype, positions, positions_shape, positions_strides, inv_freq,
                               table_dtype, mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace_pos_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                                 rope_dtype_t dtype, const int64_t* positions,
                                                 const int64_t positions_shape[2], const int64_t positions_strides[2],
                                                 const double* inv_freq, rope_dtype_t table_dtype, int64_t mode,
                                                 const int64_t partial_slice[2], void* stream)
{
    return rope::run_pos_multi(count, xs, x_shapes, dtype, positions, positions_shape, positions_strides, inv_freq,
                               table_dtype, mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const int64_t* positions, const int64_t positions_shape[2],
                                       const int64_t positions_strides[2], const double* inv_freq,
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run_out_pos(y, x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq,
                             table_dtype, mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const int64_t* positions, const int64_t positions_shape[2],
                                       const int64_t positions_strides[2], const double* inv_freq,
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run_out_pos(y, x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq,
                             table_dtype, mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_inplace_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                             rope_dtype_t dtype, const void* r1, const int64_t r1_shape[4],
                                             const int64_t r1_strides[4], const void* r2, const int64_t r2_shape[4],
                                             const int64_t r2_strides[4], rope_dtype_t table_dtype, int64_t mode,
                                             const int64_t partial_slice[2], void* stream)
{
    return rope::run_multi(count, xs, x_shapes, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                           table_dtype, mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                             rope_dtype_t dtype, const void* r1, const int64_t r1_shape[4],
                                             const int64_t r1_strides[4], const void* r2, const int64_t r2_shape[4],
                                             const int64_t r2_strides[4], rope_dtype_t table_dtype, int64_t mode,
                                             const int64_t partial_slice[2], void* stream)
{
    return rope::run_multi(count, xs, x_shapes, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                           table_dtype, mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_check(const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                 const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                 const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                 rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2])
{
    rope::Plan p;
    std::string why;
    rope_status_t st = rope::make_plan(const_cast<void*>(x), x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape,
                                       r2_strides, table_dtype, mode, partial_slice, rope::kFwd, &p, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    return ROPE_OK;
}

rope_status_t rope_partial_launch_info(const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       int64_t info[ROPE_LAUNCH_INFO_LEN])
{
    if (info == nullptr) return rope::set_error(ROPE_ERR_NULLPTR, "info is NULL");
    for (int i = 0; i < ROPE_LAUNCH_INFO_LEN; ++i) info[i] = 0;
    rope::Launch L;
    std::string why;
    rope_status_t st = rope::make_plan(const_cast<void*>(x), x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape,
                                       r2_strides, table_dtype, mode, partial_slice, rope::kFwd, &L.p, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    if (L.p.noop) return ROPE_OK;
    rope::prepare(&L);
    if (L.vec) {
        info[0] = ROPE_KERNEL_VECTOR;
        info[1] = rope::vec_grid(L.a, L.cfg);
        info[2] = (int64_t)L.a.span * L.a.HL * L.a.GL;
        info[3] = L.cfg.U;
        info[4] = L.a.HL;
        info[5] = L.a.GL;
        info[6] = L.a.xcd_group;
        info[7] = L.a.span;
    } else if (L.rows) {
        info[0] = ROPE_KERNEL_ROWS;
        info[1] = L.rs.grid;
        info[2] = L.rs.threads;
        info[4] = L.rs.rpb;
        info[7] = L.rs.tpr;
    } else {
        info[0] = ROPE_KERNEL_SCALAR;
        info[2] = 256;
    }
    return ROPE_OK;
}

rope_status_t rope_partial_launch_info_pos(const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                           const int64_t* positions, const int64_t positions_shape[2],
                                           const int64_t positions_strides[2], const double* inv_freq,
                                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                           int64_t info[ROPE_LAUNCH_INFO_LEN])
{
    if (info == nullptr) return rope::set_error(ROPE_ERR_NULLPTR, "info is NULL");
    for (int i = 0; i < ROPE_LAUNCH_INFO_LEN; ++i) info[i] = 0;
    rope::Plan p;
    std::string why;
    rope_status_t st = rope::make_plan_pos(const_cast<void*>(x), x_shape, dtype, positions, positions_shape,
                                           positions_strides, inv_freq, table_dtype, mode, partial_slice, rope::kFwd,
                                           &p, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    if (p.noop) return ROPE_OK;
    rope::PosArgs a{};
    uint32_t threads = 0, grid = 0;
    rope::RowShape rs;
    if (rope::pos_geometry(p, &a, &threads, &grid)) {
        info[0] = ROPE_KERNEL_VECTOR;
        info[1] = grid;
        info[2] = threads;
        info[3] = rope::kUPos;
        info[4] = a.HL;
        info[5] = a.P;
        info[6] = a.chunks;
        info[7] = a.span;
    } else if (rope::rows_shape(p, &rs)) {
        info[0] = ROPE_KERNEL_ROWS;
        info[1] = rs.grid;
        info[2] = rs.threads;
        info[4] = rs.rpb;
        info[7] = rs.tpr;
    } else {
        info[0] = ROPE_KERNEL_SCALAR;
        info[2] = 256;
    }
    return ROPE_OK;
}

const char* rope_status_string(rope_status_t status)
{
    switch (status) {
    case ROPE_OK: return "ROPE_OK: success";
    case ROPE_ERR_NULLPTR: return "ROPE_ERR_NULLPTR: a required pointer is NULL";
    case ROPE_ERR_INVALID: return "ROPE_ERR_INVALID: an argument violates the operation's constraints";
    case ROPE_ERR_UNSUPPORTED: return "ROPE_ERR_UNSUPPORTED: valid arguments this library does not support";
    case ROPE_ERR_RUNTIME: return "ROPE_ERR_RUNTIME: the HIP runtime reported an error";
    default: return "unknown rope_status_t";
    }
}

const char* rope_last_error(void)
{
    return rope::g_last_error.c_str();
}

}  // extern "C"
