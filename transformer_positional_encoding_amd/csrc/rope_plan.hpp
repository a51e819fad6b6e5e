// Host-side argument checking and launch planning for in-place partial RoPE.
// Pure C++ (no HIP): the checks can run, and be tested, on a machine with no
// GPU. The rules are the constraints of "CANN ops-transformer 算子详解：
// inplace_partial_rotary_mul 原地部分旋转位置编码", section 约束说明.
#pragma once

#include <stdint.h>

#include <string>

#include "rope_partial.h"

namespace rope {

enum Direction : int { kFwd = 0, kBwd = 1 };

// Everything a kernel launch needs, normalised.
struct Plan {
    int64_t B = 0, S = 0, N = 0, D = 0;
    int64_t start = 0, L = 0;
    int dtype = 0;           // rope_dtype_t of x
    int tdtype = 0;          // rope_dtype_t of r1 and r2
    int mode = 0;            // ROPE_MODE_INTERLEAVE or ROPE_MODE_ROTATE_HALF (a coefficient maps to one)
    int64_t half = 0;        // lanes between a pair's two lanes: 1 (interleave), L/2 (rotate_half) or L/c;
                             // rotate_half pairs are (g*2*half + k, g*2*half + k + half)
    int dir = kFwd;
    int esize = 0;           // bytes per element of x
    int tesize = 0;          // bytes per element of the tables
    bool noop = false;       // nothing to launch (empty tensor; in place: or empty slice)
    bool copy_only = false;  // out of place with an empty slice: y = x, no rotation
    int64_t bytes = 0;       // size of x in bytes
    void* x = nullptr;       // the tensor written (in place: also read)
    const void* src = nullptr;  // out of place: the tensor read (distinct from x); else NULL
    const void* r1 = nullptr;
    const void* r2 = nullptr;
    // Table strides in elements for the b, s and n dimensions; 0 where the
    // table broadcasts (size-1 dimension). The lane stride is 1.
    int64_t t1[3] = {0, 0, 0};
    int64_t t2[3] = {0, 0, 0};
    // Tables computed from positions (the _pos entry points) instead of
    // read: the position of (b,s) is pos[b*pos_sb + s*pos_ss] (pos_sb is 0
    // when one row of positions serves every batch); inv_freq holds L/2
    // frequencies. r1 and r2 are then NULL.
    const int64_t* pos = nullptr;
    const double* inv_freq = nullptr;
    int64_t pos_sb = 0, pos_ss = 0;
};

// Validate the C-ABI arguments in the documented order and fill `plan`.
// On failure returns the status and writes a one-line reason to `why`.
rope_status_t make_plan(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                        const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                        const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                        rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                        Direction dir, Plan* plan, std::string* why);

// Out-of-place form: y receives x with its slice rotated and x is left
// as it is. Checks, in order: the scalar arguments of make_plan; an empty
// tensor is a no-op; NULL y or x; y and x overlapping without being the
// same buffer (y == x is the in-place operation); an empty slice is a plain
// copy (the tables are not looked at); then the tables as in make_plan.
// On success plan->x is y, and plan->src is x unless y == x.
rope_status_t make_plan_out(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                            const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                            const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                            rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                            Direction dir, Plan* plan, std::string* why);

// The _pos form: cos and sin come from positions and per-pair frequencies
// (checked in place of the tables). Checks, in order: the scalar arguments
// of make_plan; an empty tensor or slice is a no-op; NULL x, positions,
// inv_freq, positions_shape or positions_strides; positions_shape is
// {1 or B, S} with strides >= 0 (a size-1 dimension's stride is ignored)
// whose offsets fit in 64 bits.
rope_status_t make_plan_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype, const int64_t* positions,
                            const int64_t positions_shape[2], const int64_t positions_strides[2],
                            const double* inv_freq, rope_dtype_t table_dtype, int64_t mode,
                            const int64_t partial_slice[2], Direction dir, Plan* plan, std::string* why);

// Out of place from positions: the checks of make_plan_out with those of
// make_plan_pos in place of the table checks (positions, frequencies,
// shape and strides), in that order.
rope_status_t make_plan_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                const int64_t* positions, const int64_t positions_shape[2],
                                const int64_t positions_strides[2], const double* inv_freq,
                                rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                Direction dir, Plan* plan, std::string* why);

// The projection with a rotary epilogue (rope_proj_fwd): y (B,S,H,Dh) =
// x (B*S, K) . w (H*Dh, K)^T, each head's slice rotated. `rope` holds y's
// geometry as a plan of the table call (x_shape = y's shape, the output
// type as its dtype, the slice, pair distance and tables).
struct ProjPlan {
    Plan rope;
    int64_t K = 0;
    int in_dtype = 0;          // rope_dtype_t of x and w (bf16 or fp16)
    int out_dtype = 0;         // rope_dtype_t of y (the inputs' type or fp32)
    const void* x = nullptr;
    const void* w = nullptr;
    void* y = nullptr;
    bool noop = false;         // y has no elements
};

// The tensors of one multi-tensor call must not share a byte: one fused
// launch rotates them all at once, so a shared byte would be read and
// written by two threads (and two rotations of one tensor would differ from
// two calls). ROPE_ERR_INVALID names the first overlapping pair.
rope_status_t check_disjoint(const Plan plans[], int n, std::string* why);

// Lanes per head the fused kernel takes: 32, 64, 96, 128 or 192 (block
// tiles of whole heads), or a multiple of 192 or 128 up to 1024 (a head over
// whole tiles).
bool proj_head_dim_supported(int64_t Dh);

// Output lanes per block tile for heads of Dh lanes: 192 when Dh is a
// multiple of 3, else 128.
int64_t proj_tile_lanes(int64_t Dh);

// With heads wider than a tile, a rotation partner must lie in the same
// tile: every group of 2*half lanes of the slice (a rotate_half pair's or a
// coefficient part pair's span) within one tile; interleave (half 1) always.
bool proj_groups_in_tiles(int64_t Dh, int64_t start, int64_t L, int64_t half);
// Whether every rotation group of every head's slice lies within one column
// tile of `tile` lanes (tiles start at multiples of `tile`; N = heads * Dh
// lanes in all): the square-tile projection kernel needs each group's
// partners in its own 256-lane tile, and its register epilogue in its own
// wave's 128 lanes.
bool proj_groups_in_column_tiles(int64_t Dh, int64_t N, int64_t start, int64_t L, int64_t half, int64_t tile);

// Checks, in order: the scalar arguments of make_plan on y's shape (with the
// output type); input type bf16 or fp16; output type the inputs' type or
// fp32; K >= 0; an empty y is a no-op; K a positive multiple of 64, Dh one
// the kernel tiles, and the slice's rotation groups within tiles
// (ROPE_ERR_UNSUPPORTED); NULL y, x or w; 16-byte
// alignment of y, x and w; sizes within 64-bit offsets; x or w of 2^31
// elements or more (ROPE_ERR_UNSUPPORTED: 32-bit offsets in the kernel); y
// overlapping x or w; then, for a non-empty slice, the tables as in
// make_plan with y's shape.
rope_status_t make_proj_plan(void* y, rope_dtype_t out_dtype, const void* x, const void* w, rope_dtype_t dtype,
                             const int64_t y_shape[4], int64_t K,
                             const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                             const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                             rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                             ProjPlan* plan, std::string* why);

int element_size(int dtype);

}  // namespace rope
