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
    int mode = 0;            // ROPE_MODE_*
    int dir = kFwd;
    int esize = 0;           // bytes per element of x
    int tesize = 0;          // bytes per element of the tables
    bool noop = false;       // empty tensor or empty slice: launch nothing
    void* x = nullptr;
    const void* r1 = nullptr;
    const void* r2 = nullptr;
    // Table strides in elements for the b, s and n dimensions; 0 where the
    // table broadcasts (size-1 dimension). The lane stride is 1.
    int64_t t1[3] = {0, 0, 0};
    int64_t t2[3] = {0, 0, 0};
};

// Validate the C-ABI arguments in the documented order and fill `plan`.
// On failure returns the status and writes a one-line reason to `why`.
rope_status_t make_plan(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                        const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                        const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                        rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                        Direction dir, Plan* plan, std::string* why);

int element_size(int dtype);

}  // namespace rope
