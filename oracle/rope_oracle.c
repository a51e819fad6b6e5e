/*
 * CPU oracle for in-place partial rotary position embedding (RoPE).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
 * baseline load this library. It shares no code, header, table or helper with
 * the HIP path, and the product never calls it.
 *
 * It is written to be checked by eye against two pages:
 *   [P1] "CANN ops-transformer 算子详解：inplace_partial_rotary_mul
 *        原地部分旋转位置编码" (inplace partial rotary mul on Ascend)
 *   [P3] "ANE实战RoPE位置编码在MIL中的纯ANE实现" (RoPE in MIL on the ANE)
 *
 * Notation. x has shape (B,S,N,D), row-major (BSND). The slice is the lane
 * range [start,end) of D; L = end - start. Inside a row, slice lane j
 * (0 <= j < L) is absolute lane start+j. c_j and s_j are r1 and r2 (cos and
 * sin) at the broadcast index of (b,s,n,j). For lane j, p(j) is its rotation
 * partner and sigma(j) is the sign of the partner term:
 *   interleave  : p(j) = j xor 1,      sigma(j) = -1 for even j, +1 for odd j
 *   rotate_half : p(j) = j +- L/2,     sigma(j) = -1 for j < L/2, +1 otherwise
 *   coefficient c (mode value c >= 2, even, dividing L): the slice splits
 *   into c parts of H = L/c lanes, and lane i of part 2k pairs with lane i
 *   of part 2k+1 ("ascend-transformer-boost 的 MlaPreprocessOperation",
 *   section 2, the rotation coefficients qRotaryCoeff / kRotaryCoeff: 2 is
 *   the half rotation; 4 and headDim are also allowed):
 *                 p(j) = j +- H,       sigma(j) = -1 in an even part, +1 in an odd one
 *   so c = 2 is rotate_half and c = L is interleave.
 * Forward  (P1, section 计算公式; P3, section 先搞懂RoPE):
 *   y_j  = x_j * c_j + sigma(j) * x_p(j) * s_j
 * Backward (P1, section 自动微分说明: the gradient of the forward, which is
 * the transpose of its Jacobian; P3, section on the backward pass: the
 * inverse rotation, which is the same thing when c and s are pair-duplicated):
 *   dx_j = g_j * c_j - sigma(j) * g_p(j) * s_p(j)
 *
 * Precision (P1, section Tiling 与 Kernel 的工程细节, mixed-precision
 * paragraph): 16-bit inputs are widened to fp32, the multiply-add runs in
 * fp32, and the result is written back with round-to-nearest-even. Here that
 * is, for 16-bit x: each product rounded to fp32, the sum rounded to fp32,
 * one RNE narrowing. With 16-bit tables the products are exact (8x8 or
 * 11x11 significand bits); with fp32 tables (P1's bf16/fp32 mixed case) their
 * rounding is part of the definition. fp32 x is evaluated in fp64 and
 * narrowed to fp32.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no contraction, so every
 * float operation below rounds exactly where it is written).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };
enum { ORACLE_ROTATE_HALF = 0, ORACLE_INTERLEAVE = 1 };
enum { ORACLE_FWD = 0, ORACLE_BWD = 1 };

/* ------------------------------------------------------------------------ */
/* 16-bit float formats, written from the IEEE 754 binary16 definition and   */
/* from bfloat16 (the upper 16 bits of binary32).                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1fu;
    uint32_t m = (uint32_t)h & 0x3ffu;
    float mag;
    if (e == 0x1fu) {
        /* infinity or NaN: same class in binary32, fraction moved to the top */
        return bits_f32((sign << 31) | 0x7f800000u | (m << 13));
    } else if (e == 0) {
        /* zero or subnormal: m * 2^-24, exact in binary32 */
        mag = ldexpf((float)m, -24);
    } else {
        /* normal: (1024 + m) * 2^(e - 15 - 10) */
        mag = ldexpf((float)(1024u + m), (int)e - 25);
    }
    return sign ? -mag : mag;
}

/* Round the non-negative integer q + rem/2^k to nearest, ties to even. */
static uint32_t round_nearest_even(uint32_t q, uint32_t rem, uint32_t k)
{
    uint32_t half = 1u << (k - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    return q;
}

uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t e32 = (u >> 23) & 0xffu;
    uint32_t m32 = u & 0x7fffffu;
    if (e32 == 0xffu) {
        if (m32 == 0)
            return (uint16_t)(sign | 0x7c00u);              /* infinity */
        return (uint16_t)(sign | 0x7e00u | (m32 >> 13));    /* quiet NaN */
    }
    /* value = sig * 2^(e32 - 127 - 23) with sig the 24-bit significand */
    int e16 = (int)e32 - 127 + 15;                           /* biased for binary16 */
    if (e16 >= 31)
        return (uint16_t)(sign | 0x7c00u);                  /* >= 2^16: overflow */
    if (e16 >= 1) {
        /* normal range: keep 10 of the 23 fraction bits, round the other 13.
           A carry out of the fraction moves into the exponent, which is the
           right encoding (and reaches infinity from the largest binade). */
        uint32_t q = ((uint32_t)e16 << 10) | (m32 >> 13);
        q = round_nearest_even(q, m32 & 0x1fffu, 13);
        return (uint16_t)(sign | q);
    }
    /* subnormal range: result is an integer count of 2^-24 */
    if (e32 == 0)
        return (uint16_t)sign;      /* binary32 zero or subnormal: below 2^-126 */
    {
        uint32_t sig = m32 | 0x800000u;                      /* 24-bit significand */
        /* count of 2^-24 units = sig * 2^(e32 - 127 - 23 + 24) = sig >> (126 - e32) */
        uint32_t shift = (uint32_t)(126 - (int)e32);         /* >= 14 here */
        if (shift > 25)
            return (uint16_t)sign;   /* below 2^-25 (half of the least subnormal) */
        uint32_t q = sig >> shift;
        uint32_t rem = sig & ((1u << shift) - 1u);
        q = round_nearest_even(q, rem, shift);
        return (uint16_t)(sign | q); /* q == 0x400 is the least normal: correct */
    }
}

/* bfloat16: the top half of binary32 (1 sign, 8 exponent, 7 fraction bits). */
float oracle_bf16_to_f32(uint16_t b)
{
    return bits_f32((uint32_t)b << 16);
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if (((u >> 23) & 0xffu) == 0xffu && (u & 0x7fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x40u);               /* NaN stays a quiet NaN */
    /* drop the low 16 bits with round-to-nearest-even; a carry ripples into
       the exponent, and from the largest finite binade into infinity */
    uint32_t q = u >> 16;
    q = round_nearest_even(q, u & 0xffffu, 16);
    return (uint16_t)q;
}

/* Bulk forms, used by the converter tests. */
void oracle_f16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(in[i]); }
void oracle_f32_to_f16_n(const float* in, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(in[i]); }
void oracle_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(in[i]); }
void oracle_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]); }

/* ------------------------------------------------------------------------ */
/* Element access                                                           */
/* ------------------------------------------------------------------------ */

static float load_f(const void* base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F32) return ((const float*)base)[idx];
    if (dtype == ORACLE_F16) return oracle_f16_to_f32(((const uint16_t*)base)[idx]);
    return oracle_bf16_to_f32(((const uint16_t*)base)[idx]);
}

static void store_f(void* base, int64_t idx, int dtype, float v)
{
    if (dtype == ORACLE_F32) ((float*)base)[idx] = v;
    else if (dtype == ORACLE_F16) ((uint16_t*)base)[idx] = oracle_f32_to_f16(v);
    else ((uint16_t*)base)[idx] = oracle_f32_to_bf16(v);
}

/* Broadcast index into a 4-D table: a size-1 dimension always reads index 0
   (P1, section 约束说明: r1/r2 broadcast against x[..., start:end]). */
static int64_t table_index(const int64_t shape[4], const int64_t strides[4],
                           int64_t b, int64_t s, int64_t n, int64_t j)
{
    int64_t idx[4] = { b, s, n, j };
    int64_t off = 0;
    for (int k = 0; k < 4; ++k)
        off += (shape[k] == 1 ? 0 : idx[k]) * strides[k];
    return off;
}

/* A mode value of 2 or more is a rotary coefficient: defined when it is even
   and divides L (L = 0: nothing is rotated). */
static int mode_defined(int mode, int64_t L)
{
    if (mode == ORACLE_INTERLEAVE || mode == ORACLE_ROTATE_HALF) return 1;
    return mode >= 2 && mode % 2 == 0 && (L == 0 || L % mode == 0);
}

static int64_t partner(int mode, int64_t j, int64_t L)
{
    if (mode >= 2) {                                        /* parts of H lanes: 2k pairs with 2k+1 */
        const int64_t H = L / mode;
        return (j / H) % 2 == 0 ? j + H : j - H;
    }
    if (mode == ORACLE_INTERLEAVE) return j ^ 1;          /* pairs (2i, 2i+1) */
    return j < L / 2 ? j + L / 2 : j - L / 2;               /* pairs (i, i+L/2) */
}

static int sigma(int mode, int64_t j, int64_t L)
{
    if (mode >= 2) {
        const int64_t H = L / mode;
        return (j / H) % 2 == 0 ? -1 : 1;                  /* the even part takes the negated partner */
    }
    if (mode == ORACLE_INTERLEAVE) return (j % 2 == 0) ? -1 : 1;
    return j < L / 2 ? -1 : 1;
}

/* ------------------------------------------------------------------------ */
/* The operation                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Rotate the slice of some rows of x in place.
 *
 * x        host buffer of nrows rows of D elements (dtype). Row r of the
 *          buffer is row rows[r] of the full (B,S,N,D) tensor, whose flat row
 *          index is (b*S + s)*N + n. With rows == NULL the buffer is the full
 *          tensor and nrows must be B*S*N.
 * r1, r2   cos and sin tables (table_dtype), with their 4-D shapes and
 *          strides in elements; a size-1 dimension broadcasts.
 * Returns 0, or -1 on an argument this oracle does not define.
 */
int rope_oracle_rows(void* x, const int64_t x_shape[4], int dtype,
                     const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                     const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                     int table_dtype, int mode, int64_t start, int64_t end, int direction,
                     const int64_t* rows, int64_t nrows)
{
    const int64_t B = x_shape[0], S = x_shape[1], N = x_shape[2], D = x_shape[3];
    const int64_t L = end - start;
    if (!mode_defined(mode, L)) return -1;
    if (direction != ORACLE_FWD && direction != ORACLE_BWD) return -1;
    if (start < 0 || end < start || end > D || (L % 2) != 0) return -1;
    if (rows == NULL && nrows != B * S * N) return -1;
    /* P1, section 功能与计算公式: start == end rotates nothing. */
    if (L == 0 || nrows == 0) return 0;

    float xs[1024];   /* the slice of one row, widened, before any write */
    if (L > 1024) return -1;

    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t n = flat % N;
        const int64_t s = (flat / N) % S;
        const int64_t b = flat / (N * S);
        const int64_t rowbase = r * D + start;

        for (int64_t j = 0; j < L; ++j)
            xs[j] = load_f(x, rowbase + j, dtype);

        for (int64_t j = 0; j < L; ++j) {
            const int64_t pj = partner(mode, j, L);
            const int sg = sigma(mode, j, L);
            /* forward uses the tables at lane j; the backward (transpose)
               takes the partner's sine, s_p(j), and the opposite sign */
            const int64_t ti = table_index(r1_shape, r1_strides, b, s, n, j);
            const int64_t si = table_index(r2_shape, r2_strides, b, s, n,
                                           direction == ORACLE_FWD ? j : pj);
            const float c = load_f(r1, ti, table_dtype);
            const float sn = load_f(r2, si, table_dtype);
            const int sign = direction == ORACLE_FWD ? sg : -sg;
            float y;
            if (dtype == ORACLE_F32) {
                double a = (double)xs[j] * (double)c;
                double t = (double)sign * (double)xs[pj] * (double)sn;
                y = (float)(a + t);
            } else {
                float a = xs[j] * c;                 /* fp32 product */
                float t = (float)sign * xs[pj] * sn; /* fp32 product */
                y = a + t;                           /* fp32 sum */
            }
            store_f(x, rowbase + j, dtype, y);       /* RNE to the storage type */
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Cos/sin tables from positions                                            */
/* ------------------------------------------------------------------------ */

/*
 * Round a double to the nearest value of a storage type, ties to even, in
 * one step (rounding to binary32 first and then to 16 bits would round
 * twice). For binary16 and bfloat16 the value is a whole number of units in
 * the last place of its binade: ulp = 2^(e - p) for a value in
 * [2^(e-1), 2^e) with p significand bits, and never below the least
 * subnormal, 2^(emin - p + 1). rint() rounds the scaled value to an integer,
 * ties to even, in the default rounding mode; scaling by powers of two is
 * exact. Returns the rounded value as a float (exact for every value of the
 * three types); +-inf past the largest finite value, NaN for NaN.
 */
static float round_to_type(double v, int dtype)
{
    if (dtype == ORACLE_F32) return (float)v;                 /* C's conversion rounds to nearest even */
    if (v != v) return (float)v;                               /* NaN */
    const int p = dtype == ORACLE_F16 ? 11 : 8;                 /* significand bits */
    const int emin = dtype == ORACLE_F16 ? -14 : -126;          /* least normal exponent */
    const double maxf = dtype == ORACLE_F16 ? 65504.0 : ldexp(2.0 - ldexp(1.0, -7), 127);
    if (v == 0.0 || isinf(v)) return (float)v;
    int e;
    (void)frexp(v, &e);                                         /* |v| in [2^(e-1), 2^e) */
    int q = e - p;
    if (q < emin - p + 1) q = emin - p + 1;                     /* subnormal spacing */
    const double r = ldexp(rint(ldexp(v, -q)), q);
    if (fabs(r) > maxf) return v > 0 ? INFINITY : -INFINITY;
    return (float)r;                                            /* exact: r is a value of the type */
}

/*
 * The cos/sin tables that "ANE实战RoPE位置编码在MIL中的纯ANE实现", section
 * 第一步, precomputes on the host, from positions and per-pair frequencies:
 * θ = p * inv_freq[i] (the page's p / base^(2i/h), with inv_freq[i] =
 * base^(-2i/L) supplied by the caller), evaluated as the double product of
 * the position and the frequency; cos θ and sin θ in double precision,
 * rounded once to the table type. Interleave writes pair i's values to lanes
 * 2i and 2i+1, rotate_half to lanes i and i + L/2, and a rotary coefficient
 * c (parts of H = L/c lanes, numbered in lane order) to lane k of part 2g and
 * lane k of part 2g+1 for i = g*H + k.
 *
 * positions  int64; the position of (b, s) is positions[b*stride_b + s*stride_s]
 * inv_freq   L/2 doubles
 * cos_out, sin_out   contiguous (Bp, S, 1, L) tables of table_dtype
 * Returns 0, or -1 on an argument this oracle does not define.
 */
int rope_oracle_pos_tables(const int64_t* positions, int64_t Bp, int64_t S, int64_t stride_b, int64_t stride_s,
                           const double* inv_freq, int64_t L, int mode, int table_dtype,
                           void* cos_out, void* sin_out)
{
    if (L <= 0 || (L % 2) != 0 || Bp < 0 || S < 0) return -1;
    if (!mode_defined(mode, L)) return -1;
    if (table_dtype != ORACLE_F32 && table_dtype != ORACLE_F16 && table_dtype != ORACLE_BF16) return -1;
    const int64_t half = L / 2;
    for (int64_t b = 0; b < Bp; ++b) {
        for (int64_t s = 0; s < S; ++s) {
            const double p = (double)positions[b * stride_b + s * stride_s];
            const int64_t row = (b * S + s) * L;
            for (int64_t i = 0; i < half; ++i) {
                const double theta = p * inv_freq[i];
                const float c = round_to_type(cos(theta), table_dtype);
                const float sn = round_to_type(sin(theta), table_dtype);
                int64_t j0 = mode == ORACLE_INTERLEAVE ? 2 * i : i;
                int64_t j1 = mode == ORACLE_INTERLEAVE ? 2 * i + 1 : i + half;
                if (mode >= 2) {                            /* pair i = g*H + k of parts 2g, 2g+1 */
                    const int64_t H = L / mode;
                    j0 = (i / H) * 2 * H + i % H;
                    j1 = j0 + H;
                }
                store_f(cos_out, row + j0, table_dtype, c);    /* exact: c is a value of the type */
                store_f(cos_out, row + j1, table_dtype, c);
                store_f(sin_out, row + j0, table_dtype, sn);
                store_f(sin_out, row + j1, table_dtype, sn);
            }
        }
    }
    return 0;
}

/* Bulk form of the one-step rounding, used by its tests. */
void oracle_round_double_n(const double* in, float* out, int64_t n, int dtype)
{ for (int64_t i = 0; i < n; ++i) out[i] = round_to_type(in[i], dtype); }
