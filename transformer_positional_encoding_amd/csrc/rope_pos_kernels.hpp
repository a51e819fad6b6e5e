// rope_pos_kernels.hpp -- the vector kernels that compute cos/sin from positions
// (in place, out of place, several tensors).
// Included once, by rope_kernels.hip (the one translation unit of the
// library): its kernels are instantiated there, next to the host code
// that selects and launches them.
#pragma once

#include "rope_vec_kernels.hpp"

namespace rope {
namespace {

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

// (cos θ, sin θ) rounded to TT, by the double evaluation. Not inlined: the
// kernels reach it rarely (16-bit tables) and its registers would otherwise
// count in theirs.
template <int TT>
__device__ __attribute__((noinline)) float2 pos_cos_sin_double(double th)
{
    double sn, cn;
    sincos(th, &sn, &cn);
    return make_float2(round_to_type<TT>(cn), round_to_type<TT>(sn));
}

// A faster route to the same values for 16-bit tables, with Ziv's rounding
// test (cheap approximation, then a proof that it rounds as the accurate
// value would, else the accurate evaluation):
//  * θ = k π/2 + r, |r| <= π/4 + 2^-30, in double: k = rint(θ 2/π), then r =
//    θ - k (P1 + P2 + P3) with π/2 split into three doubles (159 bits), one
//    fused multiply-add per part. For |θ| <= 2^30 (|k| < 2^30) each step
//    rounds once at |r| < 0.8, so r is within 3e-16 of θ - k π/2 (1.1e-16
//    measured);
//  * sin r and cos r in fp32 from r rounded to fp32, by their Taylor series
//    to r^9 and r^10 (truncation below 2e-9 at π/4) in Horner form, the
//    sine as r + r z p(z) so that its error is relative to its value; then
//    the quadrant k mod 4 swaps and negates them. Error bounds: the sine
//    within 2.4 units of 2^-24 of |sin r| (r's rounding, the last two
//    roundings, the rest; 1.93 measured over angles from 1e-12 to 1e5), the
//    cosine within 1.1e-7 absolute (1.08 units of 2^-24 measured);
//  * each value v is kept when the ends of an interval around it that holds
//    the exact value round to one value of TT: half-width |v| 2^-21 + 2^-50
//    for a value from the sine (the 2^-50 covers the reduction; with k = 0
//    it is exact, r = θ, and the term is left out) and 2^-21
//    for one from the cosine, over three times the bounds above, each end
//    moved out by a further |v| 2^-23 so that its own fp32 rounding cannot
//    pull it inside. Values of TT and the midpoints between them are fp32
//    numbers, so if both ends round to one value every number in between
//    does too, the exact cos or sin and its double evaluation (within a
//    unit in its last place) among them. About 0.05% of bf16 values and
//    0.5% of fp16 values fail the test (they lie within the half-width of
//    a rounding midpoint) and take the double evaluation, as do angles
//    beyond 2^30 and fp32 tables.
constexpr double kPosPio2P1 = 0x1.921fb54442d18p+0;
constexpr double kPosPio2P2 = 0x1.1a62633145c07p-54;
constexpr double kPosPio2P3 = -0x1.f1976b7ed8fbcp-110;
constexpr double kPosTwoOverPi = 0x1.45f306dc9c883p-1;
constexpr double kPosFastMaxAngle = 0x1p30;
constexpr float kPosFastRel = 0x1p-21f;     // the half-widths' relative part
constexpr float kPosFastAbsSin = 0x1p-50f;  // absolute part for a value from the sine
constexpr float kPosFastAbsCos = 0x1p-21f;  // absolute part for a value from the cosine

// v rounded to TT (nearest, ties to even), as TT's bits.
template <int TT>
__device__ __forceinline__ uint32_t pos_round_bits(float v)
{
    if constexpr (TT == ROPE_DTYPE_BF16) {
        const uint32_t u = __float_as_uint(v);   // finite here
        return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    } else {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
}

template <int TT>
__device__ __forceinline__ float pos_from_bits(uint32_t b)
{
    if constexpr (TT == ROPE_DTYPE_BF16) return __uint_as_float(b << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// (cos θ, sin θ) rounded to TT for position p and frequency f.
template <int TT>
__device__ __forceinline__ float2 pos_cos_sin(int64_t p, double f)
{
    const double th = static_cast<double>(p) * f;
    if constexpr (TT != ROPE_DTYPE_F32) {
        bool ok = false;
        float2 out;
        if (fabs(th) <= kPosFastMaxAngle) {
            const double k = rint(th * kPosTwoOverPi);
            double r = th;                                   // k = 0: exact, and -0 keeps its sign
            if (k != 0.0) {
                r = fma(-k, kPosPio2P1, th);
                r = fma(-k, kPosPio2P2, r);
                r = fma(-k, kPosPio2P3, r);
            }
            const float x = static_cast<float>(r);
            const float z = x * x;
            float sp = 0x1.71de3ap-19f;                        //  1/9!
            sp = __builtin_fmaf(sp, z, -0x1.a01a02p-13f);      // -1/7!
            sp = __builtin_fmaf(sp, z, 0x1.111112p-7f);        //  1/5!
            sp = __builtin_fmaf(sp, z, -0x1.555556p-3f);       // -1/3!
            const float sr = x == 0.0f ? x : __builtin_fmaf(sp * z, x, x);   // sin(±0) = ±0 exactly
            float cp = -0x1.27e4fcp-22f;                       // -1/10!
            cp = __builtin_fmaf(cp, z, 0x1.a01a02p-16f);       //  1/8!
            cp = __builtin_fmaf(cp, z, -0x1.6c16c2p-10f);      // -1/6!
            cp = __builtin_fmaf(cp, z, 0x1.555556p-5f);        //  1/4!
            cp = __builtin_fmaf(cp, z, -0.5f);
            const float cr = __builtin_fmaf(cp, z, 1.0f);
            const int q = static_cast<int>(k) & 3;
            const float sv = (q & 1) ? cr : sr, cv = (q & 1) ? sr : cr;
            const float sn = (q & 2) ? -sv : sv;                 // sin: q 0 sr, 1 cr, 2 -sr, 3 -cr
            const float cn = ((q + 1) & 2) ? -cv : cv;           // cos: q 0 cr, 1 -sr, 2 -cr, 3 sr
            // half-widths, ends moved out by |v| 2^-23 more
            const float es = fabsf(sr) * (kPosFastRel + 0x1p-23f) + (k != 0.0 ? kPosFastAbsSin : 0.0f);
            const float ec = fabsf(cr) * 0x1p-23f + kPosFastAbsCos;
            const float e_sn = (q & 1) ? ec : es, e_cn = (q & 1) ? es : ec;
            const uint32_t cb = pos_round_bits<TT>(cn), sb = pos_round_bits<TT>(sn);
            ok = pos_round_bits<TT>(cn - e_cn) == cb && pos_round_bits<TT>(cn + e_cn) == cb &&
                 pos_round_bits<TT>(sn - e_sn) == sb && pos_round_bits<TT>(sn + e_sn) == sb;
            out = make_float2(pos_from_bits<TT>(cb), pos_from_bits<TT>(sb));
        }
        if (ok) return out;
    }
    return pos_cos_sin_double<TT>(th);
}

// ---------------------------------------------------------------------------
// Vector kernel with the tables computed from positions. A block takes P
// consecutive (b,s) positions (P > 1 only when one position's heads fill
// fewer than kPosLanes threads) and, for each, a chunk of up to HL*U heads
// (HL head lanes, U heads per thread). Its threads first load the position
// and frequency of the first (cos, sin) pair each evaluates, then issue
// their x loads, then evaluate cos and sin while x is in flight: the memory
// counter drains in issue order, so the wait for the frequency does not
// wait for x, provided every load is issued on every path (indices are
// clamped, never branched around). The values go to LDS, each pair of each
// position once per block, and each thread reads those of its lanes from
// there. The thread layout is the table kernel's: interleave with
// whole-line coverage, rotate_half as pair owner (a thread takes vector k
// of both halves); the blocks walk x in XCD runs as the table kernel's do.
// Heads per thread (kUPosLines when the rows' threads also cover vectors
// outside the slice, to fill whole lines; else 1), measured on MI355X with
// the fp32 cos/sin below, in 128-thread blocks (µs per launch, cold data,
// table call beside):
//   (16,8192,32,128) shard, slice [32,96): 1 head 302-304, 2 heads 260-261 (256-257)
//   (32,4096,16,128) GQA Q, rotate_half:   1 head 160.6-160.9, 2 heads 161.8-162.7 (163.2-163.5)
//   MLA-style slice [0,64) of 192 lanes:   1 head 95.3-96.0, 2 heads 100.6-103.3 (94.5-95.9)
//   one K head, positions shared:          1 head 13.8-13.9, 2 heads 14.2-14.4 (14.3-14.4)
// 4 or 8 heads per thread, and 64- or 256-thread blocks, were slower on all.
// ---------------------------------------------------------------------------
constexpr int kUPosLines = 2;
constexpr int kPosLds = ROPE_D_LIMIT / 2;    // (cos, sin) entries per block
constexpr uint32_t kPosLanes = 128;          // threads a position's heads fill before a block takes more positions
// In place, with the batches as heads (positions shared by the batch, few
// heads): blocks of half that width, so a small grid spreads over more
// blocks. Measured on MI355X (cold data): the single K head (32,4096,1,128)
// bf16 rotate_half 15.4 -> 14.7 us, one tensor-parallel rank's Q
// (32,4096,4,128) and K (32,4096,1,128) in one call 63.6 -> 60.1 us. Out of
// place the rotate_half rows are already 64 threads wide, and halving them
// took the single K head from 15.7 to 22.3 us.
constexpr uint32_t kPosVheadsLanes = 64;
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
    uint32_t U;              // heads per thread (the kernel's template argument)
    uint32_t lanes;          // threads per position: span * HL
    uint32_t P;              // positions per block
    uint32_t N;
    uint32_t pairs;          // L/2
    uint32_t entries;        // P * pairs
    uint32_t chunks;         // head chunks per position
    uint32_t bs;             // B*S
    uint32_t items;          // ceil(bs / P) * chunks
    // vheads: the positions are the same for every batch (batch stride 0).
    // The kernel's positions are then the S values of s (bs = S), and its
    // heads are the B*N pairs (b, n) of each s (N = B*N), head h being
    // batch h / nx and head h % nx: each s's cos and sin is evaluated once
    // for every batch, and the head slots of a thread stay full when N is
    // small. Otherwise positions are (b, s) pairs g = b*S + s.
    uint32_t vheads;
    FastDiv span_div, lanes_div, pairs_div, chunk_div, s_div, nx_div;
    // Several tensors in one launch (MULTI): N counts the heads of all of
    // them; head n of a position belongs to the last tensor q with
    // hoff[q] <= n (hoff past the last tensor is UINT32_MAX), which holds
    // nt[q] heads per position and starts at xs[q].
    v4u* xs[kMultiMax];
    uint32_t nt[kMultiMax];
    uint32_t hoff[kMultiMax];
    // XCD runs, as for the table kernels (xcd_grouped_block): blocks
    // [0, xcd_full) are renumbered so that XCD x takes blocks [xP, xP + P)
    // of each window of 8P (P = xcd_group)
    uint32_t xcd_group, xcd_full;
    FastDiv xcd_div;
};

// The block's first item under the XCD runs (a bijection of [0, gridDim.x)).
__device__ __forceinline__ uint32_t pos_first_item(const PosArgs& a)
{
    const uint32_t bid = blockIdx.x;
    if (bid >= a.xcd_full) return bid;
    const uint32_t w = fast_div(bid, a.xcd_div);
    const uint32_t l = bid - w * a.xcd_div.d;
    return w * a.xcd_div.d + (l & 7u) * a.xcd_group + (l >> 3);
}

// The offset in `pos` of position g: g = b*S + s, or, vheads, g = s.
__device__ __forceinline__ int64_t pos_offset(const PosArgs& a, uint32_t g)
{
    const uint32_t b = fast_div(g, a.s_div);
    return (int64_t)b * a.pos_sb + (int64_t)(g - b * a.s_div.d) * a.pos_ss;
}

// The row of x (b*S + s)*N + n that head nl of position g stands for.
__device__ __forceinline__ uint32_t pos_row(const PosArgs& a, uint32_t g, uint32_t nl)
{
    if (!a.vheads) return g * a.N + nl;
    const uint32_t b = fast_div(nl, a.nx_div);
    return (b * a.s_div.d + g) * a.nx_div.d + (nl - b * a.nx_div.d);
}

// The (cos, sin) entries past the first blockDim of the block's table:
// entry e is pair e % pairs of the block's position g0 + e / pairs.
template <int TT>
__device__ __forceinline__ void pos_fill_rest(const PosArgs& a, uint32_t g0, float2* cs)
{
    for (uint32_t e = threadIdx.x + blockDim.x; e < a.entries; e += blockDim.x) {
        const uint32_t q = fast_div(e, a.pairs_div);
        const uint32_t ge = g0 + q;
        if (ge >= a.bs) break;                    // later entries belong to later positions
        cs[e] = pos_cos_sin<TT>(a.pos[pos_offset(a, ge)], a.inv_freq[e - q * a.pairs]);
    }
}

// The row of head nl of position g in one tensor, or, MULTI, in the tensor
// the head belongs to; as a vector pointer with the thread's vector c.
template <bool MULTI>
__device__ __forceinline__ v4u* pos_row_vec(const PosArgs& a, uint32_t g, uint32_t nl, uint32_t c)
{
    if constexpr (!MULTI) {
        return a.x + (pos_row(a, g, nl) * a.row_vecs + c);
    } else {
        // vheads: head nl is head n of the tensors' joint range in batch b,
        // at (b, s) = (b, g); otherwise g is the (b, s) pair itself
        uint32_t n = nl, bs = g;
        if (a.vheads) {
            const uint32_t b = fast_div(nl, a.nx_div);
            n = nl - b * a.nx_div.d;
            bs = b * a.s_div.d + g;
        }
        v4u* base = a.xs[0];
        uint32_t nt = a.nt[0], ho = 0;
#pragma unroll
        for (int q = 1; q < kMultiMax; ++q) {
            const bool in = n >= a.hoff[q];
            base = in ? a.xs[q] : base;
            nt = in ? a.nt[q] : nt;
            ho = in ? a.hoff[q] : ho;
        }
        return base + ((bs * nt + (n - ho)) * a.row_vecs + c);
    }
}

template <int DT, int TT, int DIR, int MODE, bool MULTI, int U>
__global__ void __launch_bounds__(256) rope_pos_kernel(PosArgs a)
{
    __shared__ float2 cs[kPosLds];   // (cos, sin) of the block's positions, pair-major per position
    constexpr int K = Store<DT>::kLanes;
    static_assert(U == 1 || U == kUPosLines, "instantiated head counts");
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
    for (uint32_t w = pos_first_item(a); w < a.items; w += gridDim.x) {
        const uint32_t grp = fast_div(w, a.chunk_div);
        const uint32_t chunk = w - grp * a.chunks;
        const uint32_t g0 = grp * a.P;                        // the block's first position
        const uint32_t ge = g0 + eq;                          // the position of entry t
        const bool fill = t < a.entries && ge < a.bs;
        const int64_t p0 = a.pos[pos_offset(a, min(ge, a.bs - 1))];
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
        pos_fill_rest<TT>(a, g0, cs);
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
    for (uint32_t w = pos_first_item(a); w < a.items; w += gridDim.x) {
        const uint32_t grp = fast_div(w, a.chunk_div);
        const uint32_t chunk = w - grp * a.chunks;
        const uint32_t g0 = grp * a.P;                        // the block's first position
        const uint32_t ge = g0 + eq;                          // the position of entry t
        const bool fill = t < a.entries && ge < a.bs;
        const int64_t p0 = a.pos[pos_offset(a, min(ge, a.bs - 1))];
        const double f0 = a.inv_freq[ei];
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t g = g0 + pp;
        const bool pos_live = g < a.bs;
        const uint32_t gl = pos_live ? g : a.bs - 1;  // past the last position: re-read it, store nothing
        const uint32_t n0 = chunk * (a.HL * U) + hl;
        v4u xa[U], xb[U];
        uint32_t off[U];
        bool live[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t n = n0 + (uint32_t)k * a.HL;
            live[k] = pos_live && n < a.N;
            const uint32_t nl = n < a.N ? n : a.N - 1;
            const uint32_t row = pos_row(a, gl, nl) * a.row_vecs;
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
        pos_fill_rest<TT>(a, g0, cs);
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

}  // namespace
}  // namespace rope
