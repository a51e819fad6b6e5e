// Argument checking for the C ABI (see rope_plan.hpp). Order of checks:
// scalars -> no-op -> pointers -> table geometry. Every combination of
// x and table dtypes is accepted (r1 and r2 share one).
#include "rope_plan.hpp"

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

}  // namespace

rope_status_t make_plan(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                        const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                        const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                        rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                        Direction dir, Plan* plan, std::string* why)
{
    // 1. scalar arguments
    if (x_shape == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "x_shape is NULL");
    if (mode != ROPE_MODE_INTERLEAVE && mode != ROPE_MODE_ROTATE_HALF)
        return fail(ROPE_ERR_INVALID, why, "mode must be 0 (rotate_half) or 1 (interleave)");
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
    int64_t numel = 1;
    for (int k = 0; k < 4; ++k) {
        if (!mul_ok(numel, x_shape[k], &numel))
            return fail(ROPE_ERR_INVALID, why, "x has more elements than 64-bit offsets can address");
    }
    int64_t bytes;
    if (!mul_ok(numel, element_size(dtype), &bytes))
        return fail(ROPE_ERR_INVALID, why, "x byte size overflows 64 bits");

    Plan p;
    p.B = x_shape[0]; p.S = x_shape[1]; p.N = x_shape[2]; p.D = D;
    p.start = start; p.L = L;
    p.dtype = dtype; p.tdtype = table_dtype; p.mode = (int)mode; p.dir = dir;
    p.esize = element_size(dtype);
    p.tesize = element_size(table_dtype);

    // 2. no-op: nothing to rotate; pointers and tables are not looked at
    if (numel == 0 || L == 0) {
        p.noop = true;
        *plan = p;
        return ROPE_OK;
    }

    // 3. pointers
    if (x == nullptr) return fail(ROPE_ERR_NULLPTR, why, "x is NULL");
    if (r1 == nullptr) return fail(ROPE_ERR_NULLPTR, why, "r1 is NULL");
    if (r2 == nullptr) return fail(ROPE_ERR_NULLPTR, why, "r2 is NULL");
    if (r1_shape == nullptr || r1_strides == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "r1 shape or strides is NULL");
    if (r2_shape == nullptr || r2_strides == nullptr)
        return fail(ROPE_ERR_NULLPTR, why, "r2 shape or strides is NULL");

    // 4. table geometry
    rope_status_t st = check_table("r1", r1_shape, r1_strides, x_shape, L, p.t1, why);
    if (st != ROPE_OK) return st;
    st = check_table("r2", r2_shape, r2_strides, x_shape, L, p.t2, why);
    if (st != ROPE_OK) return st;

    p.x = x; p.r1 = r1; p.r2 = r2;
    *plan = p;
    return ROPE_OK;
}

}  // namespace rope
