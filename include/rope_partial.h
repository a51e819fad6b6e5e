/*
 * rope_partial.h -- C ABI of the MI355X (gfx950) in-place partial rotary
 * position embedding library, librope_partial.so.
 *
 * The operation ("CANN ops-transformer 算子详解：inplace_partial_rotary_mul
 * 原地部分旋转位置编码", sections 功能与计算公式 and 约束说明; rotate_half
 * pairing from "ANE实战RoPE位置编码在MIL中的纯ANE实现", section 先搞懂RoPE):
 *
 *   x has shape (B,S,N,D), row-major and contiguous (BSND). Only the lanes
 *   [start,end) of the last dimension are rotated, in place; every other lane
 *   keeps its bytes. With L = end - start and slice lane j in [0,L):
 *     interleave  (mode 1): partner p(j) = j xor 1,   sign s(j) = -1 if j even
 *     rotate_half (mode 0): partner p(j) = j +- L/2,  sign s(j) = -1 if j < L/2
 *     rotary coefficient (mode c >= 2, even, dividing L; "ascend-transformer-
 *     boost 的 MlaPreprocessOperation", section 2, qRotaryCoeff/kRotaryCoeff:
 *     2 is the half rotation, 4 or headDim also allowed): the slice in c
 *     parts of H = L/c lanes, lane k of part 2g paired with lane k of part
 *     2g+1: p(j) = j +- H, s(j) = -1 in an even part. c = 2 is rotate_half,
 *     c = L interleave.
 *   forward : y_j  = x_j * r1_j + s(j) * x_p(j) * r2_j
 *   backward: dx_j = g_j * r1_j - s(j) * g_p(j) * r2_p(j)
 *   (the backward is the transposed Jacobian of the forward -- the gradient
 *   with respect to x, section 自动微分说明 -- which equals rotating by -θ
 *   when the tables hold one angle per pair.)
 *   r1 (cos) and r2 (sin) are read at the broadcast index of (b,s,n,j).
 *   Arithmetic is fp32 (the page's mixed-precision paragraph: inputs are
 *   cast to fp32 for the multiply-add and written back with round-to-
 *   nearest-even). For 16-bit x each product is rounded to fp32, the sum is
 *   rounded to fp32, and the result is rounded to nearest-even to the
 *   storage type; with 16-bit tables the products are exact, so that is one
 *   rounding of the exact sum. For fp32 x the multiply-add may be fused.
 *
 * Memory: every pointer is a device pointer on the current HIP device. The
 * caller owns all memory; the library allocates nothing and keeps no state
 * but a per-device cache of the compute-unit count. Calls are asynchronous on
 * `stream` (a hipStream_t; NULL is the null stream). A call that returns an
 * error before the launch has not touched device memory.
 */
#ifndef ROPE_PARTIAL_H
#define ROPE_PARTIAL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* symbols of the C ABI; everything else in the library is hidden */
#define ROPE_API __attribute__((visibility("default")))

/*
 * Status codes. The classes follow the aclnn convention described on the
 * CANN ops-transformer page on aclnnMoeTokenUnpermuteWithEpGrad, section
 * 六、返回值与错误码 (a NULL required tensor, a parameter outside the supported
 * range, an inner error); the numbers are this library's own.
 */
typedef enum rope_status {
    ROPE_OK = 0,
    ROPE_ERR_NULLPTR = 1,      /* a required pointer is NULL                   */
    ROPE_ERR_INVALID = 2,      /* an argument breaks the constraints below     */
    ROPE_ERR_UNSUPPORTED = 3,  /* a valid combination the library does not run */
    ROPE_ERR_RUNTIME = 4       /* the HIP runtime reported an error            */
} rope_status_t;

typedef enum rope_dtype {
    ROPE_DTYPE_F32 = 0,
    ROPE_DTYPE_F16 = 1,
    ROPE_DTYPE_BF16 = 2
} rope_dtype_t;

/* rotary modes; interleave keeps the integer the CANN interface gives it.
 * A mode value c >= 2 is a rotary coefficient (above). */
#define ROPE_MODE_ROTATE_HALF 0
#define ROPE_MODE_INTERLEAVE 1

/* largest supported head dimension D (the page's D limit) */
#define ROPE_D_LIMIT 1024

/* ======================== cos/sin from tables ======================== */

/*
 * rope_partial_fwd_inplace -- rotate x[..., start:end) in place (forward).
 *
 *   x            device buffer of B*S*N*D elements of `dtype`, contiguous
 *                BSND; 16-byte alignment enables the vector kernels.
 *   x_shape      host array {B, S, N, D}; each >= 0, D even, D <= 1024.
 *   dtype        storage type of x.
 *   r1, r2       device buffers: cos and sin tables of `table_dtype`.
 *   r*_shape     host arrays, 4-D; r*_shape[3] == L and, for k < 3,
 *                r*_shape[k] is 1 (broadcast) or x_shape[k]. This admits the
 *                layouts the page lists (BSND, B1ND, B11D, 111D, BS1D) and
 *                any other broadcast of the same rule.
 *   r*_strides   host arrays, strides in elements, each >= 0;
 *                r*_strides[3] must be 1. The stride of a size-1 dimension
 *                is ignored (this is what torch's expand() produces).
 *   table_dtype  storage type of r1 and r2 (any of the three, independent
 *                of dtype; the page's mixed case is 16-bit x with fp32
 *                tables).
 *   mode         ROPE_MODE_INTERLEAVE, ROPE_MODE_ROTATE_HALF, or a rotary
 *                coefficient c: even, >= 2, dividing L (when L > 0).
 *   partial_slice host array {start, end} or NULL, which means {0, 0}:
 *                0 <= start <= end <= D and L = end - start even.
 *   stream       hipStream_t to launch on, or NULL.
 *
 * Checks, in this order: scalar arguments (ROPE_ERR_NULLPTR for a NULL
 * x_shape, ROPE_ERR_INVALID otherwise); then an empty tensor (B*S*N*D == 0)
 * or an empty slice (L == 0) returns ROPE_OK at once without reading any
 * pointer (no-op, as the page specifies for forward and backward); then NULL
 * data or table pointers (ROPE_ERR_NULLPTR); then table shapes and strides
 * (ROPE_ERR_INVALID); finally the launch (ROPE_ERR_RUNTIME if HIP reports
 * an error). ROPE_ERR_UNSUPPORTED is not returned by this call (only
 * rope_proj_fwd returns it, for shapes its kernel does not tile).
 * Overlapping x with r1 or r2 is undefined. Results are deterministic: each
 * element is computed by one thread from the same inputs on every call.
 */
ROPE_API rope_status_t rope_partial_fwd_inplace(
    void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/*
 * rope_partial_bwd_inplace -- the backward of rope_partial_fwd_inplace:
 * x holds the incoming gradient dy on entry and dx on return (in place).
 * Arguments, checks and no-op rules are those of the forward; r1 and r2
 * receive no gradient (the page's autograd returns None for them).
 */
ROPE_API rope_status_t rope_partial_bwd_inplace(
    void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/*
 * rope_partial_fwd_out / rope_partial_bwd_out -- the same operation out of
 * place: y (dx) receives x (dy) with the lanes [start,end) rotated, forward
 * or backward as above, and every other lane copied bit for bit; x is not
 * modified. The page's autograd backward (section 自动微分说明) needs this
 * form: the incoming gradient may be shared with other consumers, so it
 * cannot be rotated in place, and one pass that reads it and writes the
 * result moves less memory than a copy followed by the in-place call.
 *
 *   y            device buffer for the result: B*S*N*D elements of `dtype`,
 *                contiguous BSND, owned by the caller. y == x is the
 *                in-place call; any other overlap of y and x is an error.
 *   x            device buffer of the input, same shape and type.
 *   Other arguments are those of rope_partial_fwd_inplace.
 *
 * Checks, in this order: the scalar arguments (as above); an empty tensor
 * returns ROPE_OK without reading any pointer; NULL y or x
 * (ROPE_ERR_NULLPTR); y and x overlapping without being equal
 * (ROPE_ERR_INVALID); an empty slice (L == 0) then copies x to y without
 * looking at the tables, which may be NULL; otherwise the table pointers
 * and geometry are checked as above. When both buffers are 16-byte aligned
 * (and the vector kernel's size limits hold) one kernel reads x and writes
 * y; otherwise x is copied to y on `stream` and y is rotated in place.
 */
ROPE_API rope_status_t rope_partial_fwd_out(
    void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

ROPE_API rope_status_t rope_partial_bwd_out(
    void* dx, const void* dy, const int64_t x_shape[4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/* largest tensor count of the _multi entry points */
#define ROPE_MULTI_MAX 4

/*
 * rope_partial_fwd_inplace_multi / rope_partial_bwd_inplace_multi -- rotate
 * `count` tensors that share one pair of tables (for example the Q and K of
 * one attention layer, whose head counts differ under grouped-query
 * attention) with one call; the result is that of calling the single-tensor
 * entry point on xs[0], xs[1], ... in order on `stream`. When every tensor
 * takes the same vector kernel, all of them run in a single kernel launch
 * (one launch overhead, tables shared in cache). "ANE实战RoPE位置编码在MIL中的
 * 纯ANE实现", section 第二步, applies the same rotation to Q and to K.
 *
 *   count      0..ROPE_MULTI_MAX; 0 is a no-op.
 *   xs         host array of `count` device pointers.
 *   x_shapes   host array of `count` shapes {B, S, N, D}.
 *   Other arguments are those of rope_partial_fwd_inplace and apply to every
 *   tensor: the tables must broadcast against each tensor's slice.
 *
 * Every tensor is checked before anything is launched: on an error no
 * memory has been touched, and rope_last_error() names the tensor.
 * count outside [0, ROPE_MULTI_MAX] is ROPE_ERR_INVALID; NULL xs or x_shapes
 * with count > 0 is ROPE_ERR_NULLPTR. Tensors that share any byte (the same
 * tensor passed twice included) are ROPE_ERR_INVALID, checked after every
 * tensor's own checks and before any launch: one fused launch would read
 * and write the shared bytes from two threads at once.
 */
ROPE_API rope_status_t rope_partial_fwd_inplace_multi(
    int32_t count, void* const xs[], const int64_t x_shapes[][4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

ROPE_API rope_status_t rope_partial_bwd_inplace_multi(
    int32_t count, void* const xs[], const int64_t x_shapes[][4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/* ====================== cos/sin from positions ====================== */

/*
 * rope_partial_fwd_inplace_pos / rope_partial_bwd_inplace_pos -- the same
 * in-place operation with cos and sin computed from positions instead of
 * read from tables. "ANE实战RoPE位置编码在MIL中的纯ANE实现", section 第一步,
 * builds the tables from θ = p / base^(2i/h) for position p and pair i;
 * here, for the row (b,s,n) and the slice's pair i:
 *   θ = (double)positions[b, s] * inv_freq[i]      (one double product)
 *   c = RN_T(cos θ),  s = RN_T(sin θ)             (double precision, then
 *                                                   one rounding to nearest
 *                                                   even to table_dtype T)
 * placed as a table would hold them (interleave: lanes 2i and 2i+1;
 * rotate_half: lanes i and i + L/2). The result is that of the table entry
 * points given tables (Bp, S, 1, L) of type T with these values, up to the
 * last-bit differences of two double-precision cos/sin implementations,
 * which change a rounding to T only for values within about 2^-52 of a
 * midpoint of T.
 *
 *   positions          device int64 array; the position of (b,s) is
 *                      positions[b*positions_strides[0] + s*positions_strides[1]].
 *   positions_shape    host {Bp, S}: Bp is 1 (one row of positions for every
 *                      batch) or B, and S is x's S.
 *   positions_strides  host, in elements, each >= 0; a size-1 dimension's
 *                      stride is ignored.
 *   inv_freq           device array of L/2 doubles, pair i's frequency
 *                      (base^(-2i/L) for the page's recipe; any values, e.g.
 *                      scaled frequencies, are taken as given).
 *   table_dtype        T, the type cos and sin are rounded to (any of the
 *                      three, independent of dtype).
 *   Other arguments are those of rope_partial_fwd_inplace.
 *
 * Checks, in this order: the scalar arguments; an empty tensor or slice
 * returns ROPE_OK at once; NULL x, positions, inv_freq, positions_shape or
 * positions_strides (ROPE_ERR_NULLPTR); positions_shape not {1 or B, S}, a
 * negative stride, or offsets beyond 64 bits (ROPE_ERR_INVALID). Memory as
 * for the table entry points: asynchronous on `stream`, nothing allocated.
 */
ROPE_API rope_status_t rope_partial_fwd_inplace_pos(
    void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

ROPE_API rope_status_t rope_partial_bwd_inplace_pos(
    void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/*
 * rope_partial_fwd_out_pos / rope_partial_bwd_out_pos -- the position forms
 * out of place: y receives x with its slice rotated, cos and sin computed
 * from positions exactly as rope_partial_fwd_inplace_pos does, and x is left
 * unchanged. y == x is the in-place call. An empty slice copies x to y.
 *
 *   y, x         device buffers of B*S*N*D elements of `dtype`, contiguous
 *                BSND; y is written, x is read. With both 16-byte aligned
 *                one kernel reads x and writes y in one pass; otherwise x is
 *                copied to y and y is rotated in place.
 *   Other arguments are those of rope_partial_fwd_inplace_pos.
 *
 * Checks, in this order: the scalar arguments; an empty tensor returns
 * ROPE_OK at once; NULL y or x (ROPE_ERR_NULLPTR); y and x overlapping
 * without being the same buffer (ROPE_ERR_INVALID); an empty slice copies;
 * then the checks of positions, positions_shape, positions_strides and
 * inv_freq of the in-place form. Asynchronous on `stream`; nothing is
 * allocated.
 */
ROPE_API rope_status_t rope_partial_fwd_out_pos(
    void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

ROPE_API rope_status_t rope_partial_bwd_out_pos(
    void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/*
 * rope_partial_fwd_inplace_pos_multi / rope_partial_bwd_inplace_pos_multi
 * -- the position forms for `count` tensors that share one set of positions
 * (the Q and K of one attention layer, whose head counts may differ); the
 * result is that of calling rope_partial_fwd_inplace_pos on xs[0], xs[1],
 * ... in order on `stream`. When the tensors share B, S and D and take the
 * vector kernel, all of them run in a single launch that evaluates each
 * pair's cos and sin once per position for every tensor. "ANE实战RoPE位置编码
 * 在MIL中的纯ANE实现", section 第二步, applies the same rotation to Q and K.
 *
 *   count      0..ROPE_MULTI_MAX; 0 is a no-op.
 *   xs         host array of `count` device pointers.
 *   x_shapes   host array of `count` shapes {B, S, N, D}.
 *   Other arguments are those of rope_partial_fwd_inplace_pos and apply to
 *   every tensor: positions_shape must fit each tensor's B and S.
 *
 * Every tensor is checked before anything is launched: on an error no
 * memory has been touched, and rope_last_error() names the tensor. count
 * outside [0, ROPE_MULTI_MAX] is ROPE_ERR_INVALID; NULL xs or x_shapes with
 * count > 0 is ROPE_ERR_NULLPTR. Tensors that share any byte are
 * ROPE_ERR_INVALID, as for rope_partial_fwd_inplace_multi.
 */
ROPE_API rope_status_t rope_partial_fwd_inplace_pos_multi(
    int32_t count, void* const xs[], const int64_t x_shapes[][4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

ROPE_API rope_status_t rope_partial_bwd_inplace_pos_multi(
    int32_t count, void* const xs[], const int64_t x_shapes[][4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/* ====================== checks and launch plans ====================== */

/*
 * rope_partial_check -- run every argument check of rope_partial_fwd_inplace
 * (either direction: they are the same) and return the status it would
 * return, without launching anything or touching device memory. For callers
 * that validate ahead of time, as the page's graph-mode meta implementation
 * does at compile time (section 调用说明, graph mode). Pointers are only
 * compared with NULL.
 */
ROPE_API rope_status_t rope_partial_check(
    const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2]);

/* Kernels of the launch plan (rope_partial_launch_info). */
#define ROPE_KERNEL_NONE 0   /* no-op call: nothing is launched */
#define ROPE_KERNEL_VECTOR 1 /* 16-byte vector kernel */
#define ROPE_KERNEL_SCALAR 2 /* one thread per pair, 64-bit indexing (2^31 rows or more) */
#define ROPE_KERNEL_ROWS 3   /* one thread per pair, rows of threads, any alignment */
#define ROPE_LAUNCH_INFO_LEN 8

/*
 * rope_partial_launch_info -- the launch plan a call with these arguments
 * would use (either direction: they plan alike), for tests and profiling.
 * Runs the checks of rope_partial_check first and returns their status; on
 * ROPE_OK, info (caller-owned, ROPE_LAUNCH_INFO_LEN elements) receives:
 *   [0] ROPE_KERNEL_NONE, _VECTOR, _ROWS or _SCALAR;
 *   [1] blocks of the launch (0 for the scalar kernel, whose grid follows
 *       the device's compute-unit count at launch);
 *   [2] threads per block;
 *   vector kernel: [3] heads per thread, [4] head lanes per tile, [5] tiles
 *       per block, [6] XCD run length (consecutive blocks kept on one XCD),
 *       [7] 16-byte vectors each row's threads cover;
 *   row kernel: [4] rows per block, [7] threads per row.
 * Entries that do not apply are 0. Launches nothing and touches no memory;
 * pointers are only compared with NULL and checked for alignment.
 * NULL info is ROPE_ERR_NULLPTR.
 */
ROPE_API rope_status_t rope_partial_launch_info(
    const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    int64_t info[ROPE_LAUNCH_INFO_LEN]);

/*
 * rope_partial_launch_info_pos -- the launch plan of an in-place position
 * call (rope_partial_fwd_inplace_pos / _bwd_inplace_pos) with these arguments,
 * for tests and profiling. Runs that call's checks first and returns their
 * status; on ROPE_OK, info (caller-owned, ROPE_LAUNCH_INFO_LEN elements)
 * receives:
 *   [0] ROPE_KERNEL_NONE, _VECTOR, _ROWS or _SCALAR;
 *   [1] blocks of the launch (0 for the scalar kernel);
 *   [2] threads per block;
 *   vector kernel: [3] heads per thread, [4] head lanes per position,
 *       [5] positions per block, [6] head chunks per position, [7] 16-byte
 *       vectors each row's threads cover;
 *   row kernel: [4] rows per block, [7] threads per row.
 * Entries that do not apply are 0. Launches nothing and touches no memory;
 * pointers are only compared with NULL and checked for alignment. NULL
 * info is ROPE_ERR_NULLPTR.
 */
ROPE_API rope_status_t rope_partial_launch_info_pos(
    const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
    const int64_t* positions, const int64_t positions_shape[2], const int64_t positions_strides[2],
    const double* inv_freq, rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    int64_t info[ROPE_LAUNCH_INFO_LEN]);

/* ===================== projection with a rotary epilogue ===================== */

/*
 * rope_proj_fwd -- a head projection whose epilogue rotates each head's
 * slice before the result is stored: for every token m = b*S + s and output
 * lane n = h*Dh + j,
 *     p[m,n] = fl32( sum_k x[m,k] * w[n,k] )            (fp32 accumulation)
 *     y[b,s,h,j] = p rotated on the lanes [start,end) of each head, forward,
 *                  as rope_partial_fwd_inplace rotates fp32 data, then
 *                  rounded once to y's type.
 * This is the Q projection and RoPE stages of "ascend-transformer-boost 的
 * MlaPreprocessOperation：MLA 预处理四阶段融合算子深度解析", section 3 (the
 * WUQ matmul gives headNum x 192 lanes per token; Q[..., :qRopeDim] is then
 * rotated with cos/sin of shape [tokenNum, 64] given from outside) and
 * section 2 (qRopeDim, qRotaryCoeff), fused so that the projection result is
 * rotated in registers: it is never rounded to the storage type, and never
 * written and read back, before the rotation. The quantisation, RMS norms
 * and KV-cache stages of that page are not part of this call.
 *
 *   y            device buffer of the result, (B, S, H, Dh) contiguous, of
 *                type y_dtype; owned by the caller; must not overlap x or w.
 *   y_dtype      the type of x and w, or ROPE_DTYPE_F32 (no final rounding).
 *   x            device buffer (B*S, K), row-major, of `dtype`.
 *   w            device buffer (H*Dh, K), row-major, of `dtype`: output lanes
 *                by inputs, as a linear layer stores its weight (the page's
 *                transposed-weight default).
 *   dtype        ROPE_DTYPE_BF16 or ROPE_DTYPE_F16.
 *   y_shape      host array {B, S, H, Dh}.
 *   K            inputs per token: a positive multiple of 64.
 *   r1, r2, shapes and strides, table_dtype, mode, partial_slice
 *                as for rope_partial_fwd_inplace, against y's shape: tables
 *                (1 or B, 1 or S, 1 or H, L); the page's case is one row per
 *                token, (B, S, 1, L) or (1, S, 1, L) broadcast over B.
 *   stream       hipStream_t to launch on, or NULL.
 *
 * Checks, in this order: the scalar arguments of rope_partial_fwd_inplace
 * on y's shape with y_dtype (ROPE_ERR_NULLPTR for a NULL y_shape,
 * ROPE_ERR_INVALID otherwise); dtype bf16 or fp16, y_dtype dtype or fp32
 * and K >= 0 (ROPE_ERR_INVALID); an empty y returns ROPE_OK without reading
 * any pointer; K not a positive multiple of 64; Dh not one of 32, 64, 96,
 * 128 and 192 (block tiles of whole heads) nor a multiple of 192 or 128 up
 * to 1024 (a head over whole tiles of 192 or 128 lanes, such as MLA's 576-
 * lane compressed KV with its 64 rope lanes); or, for such a wide head, a
 * rotate_half or coefficient group of the slice (2 x its pair distance
 * lanes) that spans two tiles, unless K is a multiple of 128 and every
 * group lies in one 256-lane column tile of y (ROPE_ERR_UNSUPPORTED);
 * NULL y, x or w (ROPE_ERR_NULLPTR); y, x or w not 16-byte aligned or
 * sizes beyond 64-bit offsets (ROPE_ERR_INVALID); x or w of 2^31 elements
 * or more (ROPE_ERR_UNSUPPORTED); y overlapping x or w (ROPE_ERR_INVALID); then,
 * for a non-empty slice, the tables as for rope_partial_fwd_inplace; a grid
 * too large for one launch (ROPE_ERR_UNSUPPORTED); finally the launch
 * (ROPE_ERR_RUNTIME). An empty slice gives the plain projection. The
 * library allocates nothing; results are deterministic (each output is
 * accumulated by one wave in a fixed order).
 */
ROPE_API rope_status_t rope_proj_fwd(
    void* y, rope_dtype_t y_dtype, const void* x, const void* w, rope_dtype_t dtype,
    const int64_t y_shape[4], int64_t K,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    void* stream);

/* Kernels of a projection's launch plan (rope_proj_launch_info). */
#define ROPE_KERNEL_PROJ_HEADS 4  /* tiles of whole heads: 384 x 192 (12 waves) or 256 x 128 (8 waves) */
#define ROPE_KERNEL_PROJ_SQUARE 5 /* 256 x 256 tiles, 4 waves of 128 x 128 */

/*
 * rope_proj_launch_info -- the launch plan rope_proj_fwd would use for
 * these arguments (y, x and w themselves aside), for tests and profiling.
 * Runs rope_proj_fwd's checks, with stand-ins for the y, x and w pointers
 * that pass the NULL, alignment and overlap checks, and returns their
 * status; on ROPE_OK, info (caller-owned, ROPE_LAUNCH_INFO_LEN elements)
 * receives:
 *   [0] ROPE_KERNEL_NONE (an empty y), ROPE_KERNEL_PROJ_HEADS or
 *       ROPE_KERNEL_PROJ_SQUARE (K a multiple of 128 and every rotation
 *       group of the slice inside one 256-lane column tile);
 *   [1] blocks; [2] threads per block; [3] tokens and [4] output lanes per
 *       block tile;
 *   square tiles: [5] the epilogue: 0 the general one (any geometry), 1 the
 *       vector epilogue with rotation partners in the 8-lane vector
 *       (interleave, or no slice), 2 the vector epilogue with partners whole
 *       vectors away inside one wave's 128 lanes; [6] 1 when the tables' rows
 *       are staged in LDS during the K loop (both tables shared by all heads,
 *       a row of L values 16, 32, 64 or 128 bytes).
 * Entries that do not apply are 0. Launches nothing and touches no memory;
 * table pointers are only compared with NULL and checked for alignment.
 * NULL info is ROPE_ERR_NULLPTR.
 */
ROPE_API rope_status_t rope_proj_launch_info(
    rope_dtype_t y_dtype, rope_dtype_t dtype, const int64_t y_shape[4], int64_t K,
    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
    int64_t info[ROPE_LAUNCH_INFO_LEN]);

/* ============================== status ============================== */

/* Static text for a status code; never NULL. */
ROPE_API const char* rope_status_string(rope_status_t status);

/* Text describing the last non-OK status returned on the calling thread
 * (which check failed, or the HIP error); "" if none. The pointer stays valid
 * until the next call on that thread. */
ROPE_API const char* rope_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_PARTIAL_H */
