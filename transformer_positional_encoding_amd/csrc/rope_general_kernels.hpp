// rope_general_kernels.hpp -- the general kernels (any alignment, start parity and
// slice length): the row kernel and the 64-bit scalar kernel, with tables
// or positions.
// Included once, by rope_kernels.hip (the one translation unit of the
// library): its kernels are instantiated there, next to the host code
// that selects and launches them.
#pragma once

#include "rope_pos_kernels.hpp"

namespace rope {
namespace {

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

}  // namespace
}  // namespace rope
