// Argument checking for the C ABI (see rope_plan.hpp). Order of checks:
// scalars -> no-op -> pointers -> table geometry. Every combination of
// x and table dtypes is accepted (r1 and r2 share one).
#include "rope_plan.hpp"

#include <algorithm>
#include <limits>

namespace rope {

int element_size(int dtype)
{
    switch (dtype) {
    case ROPE_DTYPE_F32: return 4;
    case ROPE_DTYPE_F16: return 2;
    case ROPE_DTYPE_BF16: return 2;
    default: return 0;
    }
}

namespace {

// a*b without signed overflow; false if it would exceed INT64_MAX
bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
    *out = a * b;
    return true;
}

rope_status_t fail(rope_status_t st, std::string* why, const std::string& msg)
{
    if (why) *why = msg;
    return st;
}

const char* kDimName[4] = {"B", "S", "N", "D"};

rope_status_t check_table(const char* name, const int64_t shape[4], const int64_t strides[4],
                          const int64_t x_shape[4], int64_t L, int64_t t[3], std::string* why)
{
    if (shape[3] != L)
        return fail(ROPE_ERR_INVALID, why,
                    std::string(name) + ": last dimension must equal the slice length end-start ("
                        + std::to_string(L) + "), got " + std::to_string(shape[3]));
    for (int k = 0; k < 3; ++k) {
        if (shape[k] != 1 && shape[k] != x_shape[k])
            return fail(ROPE_ERR_INVALID, why,
                        std::string(name) + ": dimension " + kDimName[k] + " is "
                            + std::to_string(shape[k]) + ", must be 1 or " + std::to_string(x_shape[k]));
    }
    for (int k = 0; k < 4; ++k) {
        if (strides[k] < 0)
            return fail(ROPE_ERR_INVALID, why, std::string(name) + ": negative stride");
    }
    if (strides[3] != 1)
        return fail(ROPE_ERR_INVALID, why, std::string(name) + ": the last dimension must have stride 1");
    // Largest element offset must fit; size-1 dimensions contribute nothing.
    int64_t span = L - 1;
    for (int k = 0; k < 3; ++k) {
        t[k] = shape[k] == 1 ? 0 : strides[k];
        int64_t part;
        if (!mul_ok(t[k], shape[k] - 1, &part) || span > std::numeric_limits<int64_t>::max() - part)
            return fail(ROPE_ERR_INVALID, why, std::string(name) + ": strides overflow 64-bit offsets");
        span += part;
    }
    return ROPE_OK;
}

// Check 1: the scalar arguments. Fills every field of p but the pointers.
rope_status_t check_scalars(const int64_t x_shape[4], rope_dtype_t dtype, rope_dtype_t table_dtype, int64_t mode,
                            const int64_t partial_slice[2], Direction dir, Plan* p, int64_t* numel_out,
                            std::string* why)
{
    if (x_shape == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "x_shape is NULL");
    if (mode != ROPE_MODE_INTERLEAVE && mode != ROPE_MODE_ROTATE_HALF && !(mode >= 2 && mode % 2 == 0))
        return fail(ROPE_ERR_INVALID, why,
                    "mode must be 0 (rotate_half), 1 (interleave) or an even rotary coefficient >= 2");
    if (element_size(dtype) == 0)
        return fail(ROPE_ERR_INVALID, why, "unknown dtype");
    if (element_size(table_dtype) == 0)
        return fail(ROPE_ERR_INVALID, why, "unknown table dtype");
    for (int k = 0; k < 4; ++k) {
        if (x_shape[k] < 0)
            return fail(ROPE_ERR_INVALID, why, std::string("x dimension ") + kDimName[k] + " is negative");
    }
    const int64_t D = x_shape[3];
    if (D % 2 != 0)
        return fail(ROPE_ERR_INVALID, why, "D must be even");
    if (D > ROPE_D_LIMIT)
        return fail(ROPE_ERR_INVALID, why, "D exceeds 1024");
    const int64_t start = partial_slice ? partial_slice[0] : 0;
    const int64_t end = partial_slice ? partial_slice[1] : 0;
    if (start < 0 || end < 0)
        return fail(ROPE_ERR_INVALID, why, "partial_slice bounds must be >= 0");
    if (end < start)
        return fail(ROPE_ERR_INVALID, why, "partial_slice end must be >= start");
    if (end > D)
        return fail(ROPE_ERR_INVALID, why, "partial_slice end must be <= D");
    const int64_t L = end - start;
    if (L % 2 != 0)
        return fail(ROPE_ERR_INVALID, why, "slice length end-start must be even");
    if (mode >= 2 && L % mode != 0)
        return fail(ROPE_ERR_INVALID, why, "the rotary coefficient must divide the slice length end-start");
    int64_t numel = 1;
    for (int k = 0; k < 4; ++k) {
        if (!mul_ok(numel, x_shape[k], &numel))
            return fail(ROPE_ERR_INVALID, why, "x has more elements than 64-bit offsets can address");
    }
    int64_t bytes;
    if (!mul_ok(numel, element_size(dtype), &bytes))
        return fail(ROPE_ERR_INVALID, why, "x byte size overflows 64 bits");

    p->B = x_shape[0]; p->S = x_shape[1]; p->N = x_shape[2]; p->D = D;
    p->start = start; p->L = L;
    p->dtype = dtype; p->tdtype = table_dtype; p->dir = dir;
    // A rotary coefficient c pairs lanes H = L/c apart within groups of 2H
    // lanes: H = 1 is interleave and H = L/2 rotate_half. The plan keeps the
    // two schemes, with `half` the pair distance.
    if (mode == ROPE_MODE_INTERLEAVE) {
        p->mode = ROPE_MODE_INTERLEAVE; p->half = 1;
    } else if (mode == ROPE_MODE_ROTATE_HALF) {
        p->mode = ROPE_MODE_ROTATE_HALF; p->half = L / 2;
    } else {
        p->half = L / mode;
        p->mode = p->half == 1 ? ROPE_MODE_INTERLEAVE : ROPE_MODE_ROTATE_HALF;
    }
    p->esize = element_size(dtype);
    p->tesize = element_size(table_dtype);
    p->bytes = bytes;
    *numel_out = numel;
    return ROPE_OK;
}

// Checks 3 (table pointers) and 4 (table geometry).
rope_status_t check_tables(const int64_t x_shape[4],
                           const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                           const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                           Plan* p, std::string* why)
{
    if (r1 == nullptr) return fail(ROPE_ERR_NULLPTR, why, "r1 is NULL");
    if (r2 == nullptr) return fail(ROPE_ERR_NULLPTR, why, "r2 is NULL");
    if (r1_shape == nullptr || r1_strides == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "r1 shape or strides is NULL");
    if (r2_shape == nullptr || r2_strides == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "r2 shape or strides is NULL");
    rope_status_t st = check_table("r1", r1_shape, r1_strides, x_shape, p->L, p->t1, why);
    if (st != ROPE_OK) return st;
    st = check_table("r2", r2_shape, r2_strides, x_shape, p->L, p->t2, why);
    if (st != ROPE_OK) return st;
    p->r1 = r1;
    p->r2 = r2;
    return ROPE_OK;
}

}  // namespace

rope_status_t make_plan(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                        const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                        const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                        rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                        Direction dir, Plan* plan, std::string* why)
{
    // 1. scalar arguments
    Plan p;
    int64_t numel = 0;
    rope_status_t st = check_scalars(x_shape, dtype, table_dtype, mode, partial_slice, dir, &p, &numel, why);
    if (st != ROPE_OK) return st;

    // 2. no-op: nothing to rotate; pointers and tables are not looked at
    if (numel == 0 || p.L == 0) {
        p.noop = true;
        *plan = p;
        return ROPE_OK;
    }

    // 3./4. pointers and table geometry
    if (x == nullptr) return fail(ROPE_ERR_NULLPTR, why, "x is NULL");
    st = check_tables(x_shape, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, &p, why);
    if (st != ROPE_OK) return st;
    p.x = x;
    *plan = p;
    return ROPE_OK;
}

rope_status_t make_plan_out(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                            const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                            const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                            rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                            Direction dir, Plan* plan, std::string* why)
{
    Plan p;
    int64_t numel = 0;
    rope_status_t st = check_scalars(x_shape, dtype, table_dtype, mode, partial_slice, dir, &p, &numel, why);
    if (st != ROPE_OK) return st;
    if (numel == 0) {
        p.noop = true;
        *plan = p;
        return ROPE_OK;
    }
    if (y == nullptr) return fail(ROPE_ERR_NULLPTR, why, "y is NULL");
    if (x == nullptr) return fail(ROPE_ERR_NULLPTR, why, "x is NULL");
    // [y, y+bytes) and [x, x+bytes) overlap iff either start lies less than
    // `bytes` past the other (unsigned differences; no pointer arithmetic)
    const uintptr_t yu = reinterpret_cast<uintptr_t>(y), xu = reinterpret_cast<uintptr_t>(x);
    const uint64_t nb = (uint64_t)p.bytes;
    const bool same = yu == xu;
    if (!same && ((uint64_t)(yu - xu) < nb || (uint64_t)(xu - yu) < nb))
        return fail(ROPE_ERR_INVALID, why, "y and x overlap without being the same buffer");
    if (p.L == 0) {
        // y = x: a copy, or nothing at all when they are one buffer
        p.noop = same;
        p.copy_only = !same;
    } else {
        st = check_tables(x_shape, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, &p, why);
        if (st != ROPE_OK) return st;
    }
    p.x = y;
    p.src = same ? nullptr : x;
    *plan = p;
    return ROPE_OK;
}

// The positions and frequencies of the _pos entry points (after the no-op
// test): pointers, the {1 or B, S} shape, non-negative strides and 64-bit
// offsets. Fills p's position fields.
static rope_status_t check_positions(const int64_t x_shape[4], const int64_t* positions,
                                     const int64_t positions_shape[2], const int64_t positions_strides[2],
                                     const double* inv_freq, Plan* p, std::string* why)
{
    if (positions == nullptr) return fail(ROPE_ERR_NULLPTR, why, "positions is NULL");
    if (inv_freq == nullptr) return fail(ROPE_ERR_NULLPTR, why, "inv_freq is NULL");
    if (positions_shape == nullptr || positions_strides == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "positions shape or strides is NULL");
    if (positions_shape[0] != 1 && positions_shape[0] != x_shape[0])
        return fail(ROPE_ERR_INVALID, why, "positions: dimension B is " + std::to_string(positions_shape[0])
                                               + ", must be 1 or " + std::to_string(x_shape[0]));
    if (positions_shape[1] != x_shape[1])
        return fail(ROPE_ERR_INVALID, why, "positions: dimension S is " + std::to_string(positions_shape[1])
                                               + ", must be " + std::to_string(x_shape[1]));
    if (positions_strides[0] < 0 || positions_strides[1] < 0)
        return fail(ROPE_ERR_INVALID, why, "positions: negative stride");
    const int64_t sb = positions_shape[0] == 1 ? 0 : positions_strides[0];
    const int64_t ss = positions_shape[1] == 1 ? 0 : positions_strides[1];
    int64_t part_b, part_s;
    if (!mul_ok(sb, positions_shape[0] - 1, &part_b) || !mul_ok(ss, positions_shape[1] - 1, &part_s) ||
        part_b > std::numeric_limits<int64_t>::max() - part_s)
        return fail(ROPE_ERR_INVALID, why, "positions: strides overflow 64-bit offsets");
    p->pos = positions;
    p->inv_freq = inv_freq;
    p->pos_sb = sb;
    p->pos_ss = ss;
    return ROPE_OK;
}

rope_status_t make_plan_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype, const int64_t* positions,
                            const int64_t positions_shape[2], const int64_t positions_strides[2],
                            const double* inv_freq, rope_dtype_t table_dtype, int64_t mode,
                            const int64_t partial_slice[2], Direction dir, Plan* plan, std::string* why)
{
    Plan p;
    int64_t numel = 0;
    rope_status_t st = check_scalars(x_shape, dtype, table_dtype, mode, partial_slice, dir, &p, &numel, why);
    if (st != ROPE_OK) return st;
    if (numel == 0 || p.L == 0) {
        p.noop = true;
        *plan = p;
        return ROPE_OK;
    }
    if (x == nullptr) return fail(ROPE_ERR_NULLPTR, why, "x is NULL");
    st = check_positions(x_shape, positions, positions_shape, positions_strides, inv_freq, &p, why);
    if (st != ROPE_OK) return st;
    p.x = x;
    *plan = p;
    return ROPE_OK;
}

rope_status_t make_plan_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                const int64_t* positions, const int64_t positions_shape[2],
                                const int64_t positions_strides[2], const double* inv_freq,
                                rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                Direction dir, Plan* plan, std::string* why)
{
    Plan p;
    int64_t numel = 0;
    rope_status_t st = check_scalars(x_shape, dtype, table_dtype, mode, partial_slice, dir, &p, &numel, why);
    if (st != ROPE_OK) return st;
    if (numel == 0) {
        p.noop = true;
        *plan = p;
        return ROPE_OK;
    }
    if (y == nullptr) return fail(ROPE_ERR_NULLPTR, why, "y is NULL");
    if (x == nullptr) return fail(ROPE_ERR_NULLPTR, why, "x is NULL");
    const uintptr_t yu = reinterpret_cast<uintptr_t>(y), xu = reinterpret_cast<uintptr_t>(x);
    const uint64_t nb = (uint64_t)p.bytes;
    const bool same = yu == xu;
    if (!same && ((uint64_t)(yu - xu) < nb || (uint64_t)(xu - yu) < nb))
        return fail(ROPE_ERR_INVALID, why, "y and x overlap without being the same buffer");
    if (p.L == 0) {
        p.noop = same;
        p.copy_only = !same;
    } else {
        st = check_positions(x_shape, positions, positions_shape, positions_strides, inv_freq, &p, why);
        if (st != ROPE_OK) return st;
    }
    p.x = y;
    p.src = same ? nullptr : x;
    *plan = p;
    return ROPE_OK;
}

rope_status_t check_disjoint(const Plan plans[], int n, std::string* why)
{
    for (int i = 0; i < n; ++i) {
        const uintptr_t ai = reinterpret_cast<uintptr_t>(plans[i].x);
        for (int j = i + 1; j < n; ++j) {
            const uintptr_t aj = reinterpret_cast<uintptr_t>(plans[j].x);
            // [ai, ai+bi) and [aj, aj+bj) overlap iff either start lies inside the other
            const bool overlap = (ai >= aj && (uint64_t)(ai - aj) < (uint64_t)plans[j].bytes) ||
                                 (aj >= ai && (uint64_t)(aj - ai) < (uint64_t)plans[i].bytes);
            if (overlap)
                return fail(ROPE_ERR_INVALID, why, "tensors " + std::to_string(i) + " and " + std::to_string(j)
                                                       + " overlap");
        }
    }
    return ROPE_OK;
}

bool proj_head_dim_supported(int64_t Dh)
{
    if (Dh == 32 || Dh == 64 || Dh == 96 || Dh == 128 || Dh == 192) return true;   // whole heads per tile
    return Dh > 192 && Dh <= ROPE_D_LIMIT && (Dh % 192 == 0 || Dh % 128 == 0);   // a head over whole tiles
}

int64_t proj_tile_lanes(int64_t Dh) { return Dh % 3 == 0 ? 192 : 128; }

bool proj_groups_in_tiles(int64_t Dh, int64_t start, int64_t L, int64_t half)
{
    const int64_t bn = proj_tile_lanes(Dh);
    if (Dh <= bn || L == 0 || half == 1) return true;   // whole heads per tile, or pairs of adjacent lanes
    for (int64_t lo = start; lo < start + L; lo += 2 * half)
        if (lo / bn != (lo + 2 * half - 1) / bn) return false;
    return true;
}

bool proj_groups_in_column_tiles(int64_t Dh, int64_t N, int64_t start, int64_t L, int64_t half, int64_t kTile)
{
    if (L == 0) return true;
    const int64_t g = 2 * half;                        // lanes per rotation group
    if (g > kTile) return false;
    // groups on a grid of g lanes in every head never straddle a tile edge
    if (kTile % g == 0 && start % g == 0 && Dh % g == 0) return true;
    // head h's groups start at h*Dh + start + j*g; the offsets mod kTile
    // repeat after kTile / gcd(Dh, kTile) heads
    int64_t a = Dh, b = kTile;
    while (b != 0) { const int64_t r = a % b; a = b; b = r; }
    const int64_t heads = std::min(N / Dh, kTile / a);
    for (int64_t h = 0; h < heads; ++h)
        for (int64_t lo = h * Dh + start; lo < h * Dh + start + L; lo += g)
            if (lo / kTile != (lo + g - 1) / kTile) return false;
    return true;
}

rope_status_t make_proj_plan(void* y, rope_dtype_t out_dtype, const void* x, const void* w, rope_dtype_t dtype,
                             const int64_t y_shape[4], int64_t K,
                             const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                             const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                             rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                             ProjPlan* plan, std::string* why)
{
    ProjPlan q;
    int64_t numel = 0;
    rope_status_t st = check_scalars(y_shape, out_dtype, table_dtype, mode, partial_slice, kFwd, &q.rope, &numel, why);
    if (st != ROPE_OK) return st;
    if (dtype != ROPE_DTYPE_BF16 && dtype != ROPE_DTYPE_F16)
        return fail(ROPE_ERR_INVALID, why, "the projection takes bf16 or fp16 x and w");
    if (out_dtype != dtype && out_dtype != ROPE_DTYPE_F32)
        return fail(ROPE_ERR_INVALID, why, "y must have the type of x and w, or fp32");
    if (K < 0) return fail(ROPE_ERR_INVALID, why, "K is negative");
    q.K = K;
    q.in_dtype = dtype;
    q.out_dtype = out_dtype;
    if (numel == 0) {
        q.noop = true;
        *plan = q;
        return ROPE_OK;
    }
    const int64_t Dh = y_shape[3];
    if (K == 0 || K % 64 != 0)
        return fail(ROPE_ERR_UNSUPPORTED, why, "K must be a positive multiple of 64");
    if (!proj_head_dim_supported(Dh))
        return fail(ROPE_ERR_UNSUPPORTED, why,
                    "head dimension must be 32, 64, 96, 128 or 192, or a multiple of 192 or 128 up to 1024");
    // a rotation group must lie in one column tile of the kernel that takes
    // the call: a tile of whole heads (or of part of a wider head), or, with
    // K a multiple of 128, a 256-lane square tile
    if (!proj_groups_in_tiles(Dh, q.rope.start, q.rope.L, q.rope.half) &&
        !(K % 128 == 0 && proj_groups_in_column_tiles(Dh, y_shape[2] * Dh, q.rope.start, q.rope.L, q.rope.half, 256)))
        return fail(ROPE_ERR_UNSUPPORTED, why,
                    "a rotation group of the slice spans two column tiles of a head wider than the tile");
    if (y == nullptr) return fail(ROPE_ERR_NULLPTR, why, "y is NULL");
    if (x == nullptr) return fail(ROPE_ERR_NULLPTR, why, "x is NULL");
    if (w == nullptr) return fail(ROPE_ERR_NULLPTR, why, "w is NULL");
    const auto misaligned = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
    if (misaligned(y) || misaligned(x) || misaligned(w))
        return fail(ROPE_ERR_INVALID, why, "y, x and w must be 16-byte aligned");
    const int64_t M = y_shape[0] * y_shape[1];   // no overflow: numel fits and the other factors are >= 1
    const int64_t N = y_shape[2] * Dh;
    int64_t x_bytes, w_bytes;
    if (!mul_ok(M, K, &x_bytes) || !mul_ok(x_bytes, 2, &x_bytes) || !mul_ok(N, K, &w_bytes) ||
        !mul_ok(w_bytes, 2, &w_bytes))
        return fail(ROPE_ERR_INVALID, why, "x or w byte size overflows 64 bits");
    // the kernel addresses x and w with 32-bit element offsets
    if (M * K >= (int64_t(1) << 31) || N * K >= (int64_t(1) << 31))
        return fail(ROPE_ERR_UNSUPPORTED, why, "x and w must each hold fewer than 2^31 elements");
    const auto overlap = [](const void* a, uint64_t na, const void* b, uint64_t nb) {
        const uintptr_t au = reinterpret_cast<uintptr_t>(a), bu = reinterpret_cast<uintptr_t>(b);
        return (au >= bu && (uint64_t)(au - bu) < nb) || (bu >= au && (uint64_t)(bu - au) < na);
    };
    const uint64_t y_bytes = (uint64_t)q.rope.bytes;
    if (overlap(y, y_bytes, x, (uint64_t)x_bytes) || overlap(y, y_bytes, w, (uint64_t)w_bytes))
        return fail(ROPE_ERR_INVALID, why, "y overlaps x or w");
    if (q.rope.L > 0) {
        st = check_tables(y_shape, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, &q.rope, why);
        if (st != ROPE_OK) return st;
    }
    q.x = x;
    q.w = w;
    q.y = y;
    q.rope.x = y;
    *plan = q;
    return ROPE_OK;
}

}  // namespace rope
