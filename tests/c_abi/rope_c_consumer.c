/*
 * A plain C client of librope_partial.so: it uses the library through the C
 * ABI declared in include/rope_partial.h and nothing else (no PyTorch, no
 * Python). Device memory and streams come from the HIP runtime API. It runs
 * the in-place, out-of-place, multi-tensor and position entry points and
 * compares every element with the CPU oracle (oracle/librope_oracle.so,
 * test infrastructure), and it checks the documented status codes.
 *
 * The operation: "CANN ops-transformer 算子详解：inplace_partial_rotary_mul
 * 原地部分旋转位置编码", sections 功能与计算公式 and 约束说明; rotate_half
 * pairing from "ANE实战RoPE位置编码在MIL中的纯ANE实现", section 先搞懂RoPE.
 *
 *   rope_c_consumer            all cases (needs a GPU)
 *   rope_c_consumer --no-gpu   only the calls that return before any HIP call
 *                              (argument errors and no-ops)
 *
 * Prints one line per case and "all ok" at the end; exits non-zero on the
 * first failure.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rope_partial.h"

/* The oracle's entry point (test infrastructure, linked for checking only):
 * rows == NULL means every row, and nrows must then be B*S*N. */
int rope_oracle_rows(void* x, const int64_t x_shape[4], int dtype,
                     const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                     const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                     int table_dtype, int mode, int64_t start, int64_t end, int direction,
                     const int64_t* rows, int64_t nrows);
/* The oracle's cos/sin tables of positions: (Bp, S, 1, L) each. */
int rope_oracle_pos_tables(const int64_t* positions, int64_t Bp, int64_t S, int64_t stride_b, int64_t stride_s,
                           const double* inv_freq, int64_t L, int mode, int table_dtype,
                           void* cos_out, void* sin_out);

#define FAIL(...) do { fprintf(stderr, "FAIL: " __VA_ARGS__); fprintf(stderr, "\n"); exit(1); } while (0)
#define HIP_OK(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_)); } while (0)

/* ---- seeded inputs (splitmix64); values, never the rotation ---- */
static uint64_t g_state;
static uint64_t next_u64(void)
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float uniform_pm1(void) { return (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0); }

/* One element of storage type dtype: fp32 in [-4, 4); a bf16 by keeping the
 * top half of such an fp32; an fp16 built from its fields (normal, |v| in
 * [2^-6, 4)). No rounding is involved in making any of them. */
static void fill(void* buf, int dtype, int64_t n, float scale)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = uniform_pm1() * scale;
        if (dtype == ROPE_DTYPE_F32) {
            ((float*)buf)[i] = f;
        } else if (dtype == ROPE_DTYPE_BF16) {
            uint32_t u;
            memcpy(&u, &f, 4);
            ((uint16_t*)buf)[i] = (uint16_t)(u >> 16);
        } else {
            uint64_t r = next_u64();
            uint16_t sign = (uint16_t)((r & 1u) << 15);
            uint16_t expo = (uint16_t)(9 + (r >> 1) % 8);      /* biased exponent 9..16 */
            uint16_t mant = (uint16_t)((r >> 8) & 0x3ffu);
            ((uint16_t*)buf)[i] = (uint16_t)(sign | (expo << 10) | mant);
        }
    }
}

static int esize(int dtype) { return dtype == ROPE_DTYPE_F32 ? 4 : 2; }
static int64_t numel4(const int64_t s[4]) { return s[0] * s[1] * s[2] * s[3]; }
static void contiguous_strides(const int64_t s[4], int64_t st[4])
{
    st[3] = 1; st[2] = s[3]; st[1] = s[2] * s[3]; st[0] = s[1] * s[2] * s[3];
}

static void* dev_copy(const void* host, size_t bytes)
{
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* Compare storage arrays: 16-bit bit for bit; fp32 within a bound scaled by
 * the largest |x| * |table| (the Python tests hold the per-lane bound). */
static void compare(const char* what, const void* got, const void* want, int dtype, int64_t n, double scale)
{
    int64_t bad = 0;
    if (dtype == ROPE_DTYPE_F32) {
        const float* g = (const float*)got;
        const float* w = (const float*)want;
        for (int64_t i = 0; i < n; ++i)
            if (!(fabs((double)g[i] - (double)w[i]) <= 2e-6 * scale)) ++bad;
    } else {
        bad = 0;
        for (int64_t i = 0; i < n; ++i)
            if (((const uint16_t*)got)[i] != ((const uint16_t*)want)[i]) ++bad;
    }
    if (bad) FAIL("%s: %lld of %lld elements differ from the oracle", what, (long long)bad, (long long)n);
    printf("ok   %s (%lld elements)\n", what, (long long)n);
}

typedef struct {
    const char* name;
    int64_t xs[4];
    int dtype, tdtype, mode, dir;
    int64_t sl[2];
    int64_t ts[4];
    int form;          /* 0 in place, 1 out of place, 2 multi (second tensor: N2 heads) */
    int64_t n2;
    int own_stream;
} Case;

static void run_case(const Case* c)
{
    const int64_t n = numel4(c->xs), tn = numel4(c->ts);
    int64_t tst[4];
    contiguous_strides(c->ts, tst);
    for (int k = 0; k < 3; ++k)
        if (c->ts[k] == 1) tst[k] = 0;   /* broadcast dimension: stride 0, as expand() gives */
    const size_t xb = (size_t)n * esize(c->dtype), tb = (size_t)tn * esize(c->tdtype);
    void* x = malloc(xb); void* r1 = malloc(tb); void* r2 = malloc(tb);
    fill(x, c->dtype, n, 4.0f);
    fill(r1, c->tdtype, tn, 1.0f);
    fill(r2, c->tdtype, tn, 1.0f);
    void* dx = dev_copy(x, xb);
    void* dr1 = dev_copy(r1, tb);
    void* dr2 = dev_copy(r2, tb);
    hipStream_t s = NULL;
    if (c->own_stream) HIP_OK(hipStreamCreate(&s));
    rope_status_t st;
    void* out = malloc(xb);
    void* want = malloc(xb);
    memcpy(want, x, xb);
    if (rope_oracle_rows(want, c->xs, c->dtype, r1, c->ts, tst, r2, c->ts, tst, c->tdtype, c->mode, c->sl[0],
                         c->sl[1], c->dir, NULL, c->xs[0] * c->xs[1] * c->xs[2]) != 0)
        FAIL("%s: the oracle rejected the case", c->name);
    const double scale = 4.0 * 4.0;
    if (c->form == 0) {
        st = (c->dir == 0 ? rope_partial_fwd_inplace : rope_partial_bwd_inplace)(
            dx, c->xs, c->dtype, dr1, c->ts, tst, dr2, c->ts, tst, c->tdtype, c->mode, c->sl, s);
        if (st != ROPE_OK) FAIL("%s: status %d (%s)", c->name, st, rope_last_error());
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(out, dx, xb, hipMemcpyDeviceToHost));
        compare(c->name, out, want, c->dtype, n, scale);
    } else if (c->form == 1) {
        void* dy = NULL;
        HIP_OK(hipMalloc(&dy, xb));
        HIP_OK(hipMemset(dy, 0xff, xb));
        st = (c->dir == 0 ? rope_partial_fwd_out : rope_partial_bwd_out)(
            dy, dx, c->xs, c->dtype, dr1, c->ts, tst, dr2, c->ts, tst, c->tdtype, c->mode, c->sl, s);
        if (st != ROPE_OK) FAIL("%s: status %d (%s)", c->name, st, rope_last_error());
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(out, dy, xb, hipMemcpyDeviceToHost));
        compare(c->name, out, want, c->dtype, n, scale);
        HIP_OK(hipMemcpy(out, dx, xb, hipMemcpyDeviceToHost));
        if (memcmp(out, x, xb) != 0) FAIL("%s: the input changed", c->name);
        HIP_OK(hipFree(dy));
    } else {
        int64_t shapes[2][4] = {{c->xs[0], c->xs[1], c->xs[2], c->xs[3]}, {c->xs[0], c->xs[1], c->n2, c->xs[3]}};
        const int64_t n2 = numel4(shapes[1]);
        const size_t xb2 = (size_t)n2 * esize(c->dtype);
        void* x2 = malloc(xb2);
        fill(x2, c->dtype, n2, 4.0f);
        void* dx2 = dev_copy(x2, xb2);
        void* want2 = malloc(xb2);
        memcpy(want2, x2, xb2);
        if (rope_oracle_rows(want2, shapes[1], c->dtype, r1, c->ts, tst, r2, c->ts, tst, c->tdtype, c->mode,
                             c->sl[0], c->sl[1], c->dir, NULL, n2 / c->xs[3]) != 0)
            FAIL("%s: the oracle rejected tensor 1", c->name);
        void* xs[2] = {dx, dx2};
        st = (c->dir == 0 ? rope_partial_fwd_inplace_multi : rope_partial_bwd_inplace_multi)(
            2, xs, (const int64_t(*)[4])shapes, c->dtype, dr1, c->ts, tst, dr2, c->ts, tst, c->tdtype, c->mode,
            c->sl, s);
        if (st != ROPE_OK) FAIL("%s: status %d (%s)", c->name, st, rope_last_error());
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(out, dx, xb, hipMemcpyDeviceToHost));
        compare(c->name, out, want, c->dtype, n, scale);
        void* out2 = malloc(xb2);
        HIP_OK(hipMemcpy(out2, dx2, xb2, hipMemcpyDeviceToHost));
        compare("  and its second tensor", out2, want2, c->dtype, n2, scale);
        free(out2); free(x2); free(want2);
        HIP_OK(hipFree(dx2));
    }
    if (s) HIP_OK(hipStreamDestroy(s));
    HIP_OK(hipFree(dx)); HIP_OK(hipFree(dr1)); HIP_OK(hipFree(dr2));
    free(x); free(r1); free(r2); free(out); free(want);
}

/* The position entry point: per-batch positions offset_b + s (offsets
 * below 2^16), frequencies base^(-2i/L) computed here in double, tables
 * computed in the kernel; the oracle builds the same tables and rotates. */
static void run_pos_case(const char* name, const int64_t xs[4], int dtype, int tdtype, int mode, int dir,
                         const int64_t sl[2], double base)
{
    const int64_t n = numel4(xs), B = xs[0], S = xs[1], L = sl[1] - sl[0];
    const size_t xb = (size_t)n * esize(dtype);
    void* x = malloc(xb);
    fill(x, dtype, n, 4.0f);
    int64_t* pos = (int64_t*)malloc((size_t)(B * S) * sizeof(int64_t));
    for (int64_t b = 0; b < B; ++b) {
        const int64_t off = (int64_t)(next_u64() % 65536u);
        for (int64_t t = 0; t < S; ++t) pos[b * S + t] = off + t;
    }
    double* f = (double*)malloc((size_t)(L / 2) * sizeof(double));
    for (int64_t i = 0; i < L / 2; ++i) f[i] = pow(base, -2.0 * (double)i / (double)L);
    const int64_t ts[4] = {B, S, 1, L};
    int64_t tst[4];
    contiguous_strides(ts, tst);
    tst[2] = 0;
    const size_t tb = (size_t)numel4(ts) * esize(tdtype);
    void* c = malloc(tb);
    void* sn = malloc(tb);
    if (rope_oracle_pos_tables(pos, B, S, S, 1, f, L, mode, tdtype, c, sn) != 0)
        FAIL("%s: the oracle rejected the positions", name);
    void* want = malloc(xb);
    memcpy(want, x, xb);
    if (rope_oracle_rows(want, xs, dtype, c, ts, tst, sn, ts, tst, tdtype, mode, sl[0], sl[1], dir, NULL,
                         B * S * xs[2]) != 0)
        FAIL("%s: the oracle rejected the case", name);
    void* dx = dev_copy(x, xb);
    void* dpos = dev_copy(pos, (size_t)(B * S) * sizeof(int64_t));
    void* df = dev_copy(f, (size_t)(L / 2) * sizeof(double));
    const int64_t pshape[2] = {B, S}, pstrides[2] = {S, 1};
    int64_t info[ROPE_LAUNCH_INFO_LEN];
    rope_status_t st = rope_partial_launch_info_pos(dx, xs, dtype, (const int64_t*)dpos, pshape, pstrides,
                                                    (const double*)df, tdtype, mode, sl, info);
    if (st != ROPE_OK || info[0] == ROPE_KERNEL_NONE) FAIL("%s: launch plan status %d", name, st);
    /* out of place first (x must stay unchanged), then in place */
    void* dy = NULL;
    HIP_OK(hipMalloc(&dy, xb));
    st = (dir == 0 ? rope_partial_fwd_out_pos : rope_partial_bwd_out_pos)(
        dy, dx, xs, dtype, (const int64_t*)dpos, pshape, pstrides, (const double*)df, tdtype, mode, sl, NULL);
    if (st != ROPE_OK) FAIL("%s, out of place: status %d (%s)", name, st, rope_last_error());
    HIP_OK(hipStreamSynchronize(NULL));
    void* out = malloc(xb);
    HIP_OK(hipMemcpy(out, dy, xb, hipMemcpyDeviceToHost));
    compare("  out of place", out, want, dtype, n, 4.0);
    HIP_OK(hipMemcpy(out, dx, xb, hipMemcpyDeviceToHost));
    if (memcmp(out, x, xb) != 0) FAIL("%s, out of place: the input changed", name);
    st = (dir == 0 ? rope_partial_fwd_inplace_pos : rope_partial_bwd_inplace_pos)(
        dx, xs, dtype, (const int64_t*)dpos, pshape, pstrides, (const double*)df, tdtype, mode, sl, NULL);
    if (st != ROPE_OK) FAIL("%s: status %d (%s)", name, st, rope_last_error());
    HIP_OK(hipStreamSynchronize(NULL));
    HIP_OK(hipMemcpy(out, dx, xb, hipMemcpyDeviceToHost));
    compare(name, out, want, dtype, n, 4.0);
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(dx)); HIP_OK(hipFree(dpos)); HIP_OK(hipFree(df));
    free(x); free(pos); free(f); free(c); free(sn); free(want); free(out);
}

/* Calls that must return before any HIP call: errors and no-ops. */
static void expect(const char* what, rope_status_t got, rope_status_t want, const char* text)
{
    if (got != want) FAIL("%s: status %d, expected %d", what, got, want);
    if (want != ROPE_OK && (strlen(rope_last_error()) == 0 || (text && !strstr(rope_last_error(), text))))
        FAIL("%s: last error '%s' does not name '%s'", what, rope_last_error(), text ? text : "");
    if (strncmp(rope_status_string(got), "ROPE_", 5) != 0) FAIL("%s: status string", what);
    printf("ok   %s -> %s\n", what, rope_status_string(got));
}

static void check_errors(void)
{
    void* fake = (void*)(uintptr_t)0x10000;       /* never dereferenced */
    void* fake_y = (void*)(uintptr_t)0x200000;
    int64_t xs[4] = {2, 4, 3, 64}, ts[4] = {1, 4, 1, 32}, tst[4] = {0, 32, 0, 1}, sl[2] = {0, 32};
    int64_t bad_sl[2] = {0, 31}, empty_sl[2] = {8, 8}, xs_empty[4] = {0, 4, 3, 64};
    expect("NULL x", rope_partial_fwd_inplace(NULL, xs, ROPE_DTYPE_BF16, fake, ts, tst, fake, ts, tst,
                                              ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_NULLPTR, "x is NULL");
    expect("mode 7", rope_partial_bwd_inplace(fake, xs, ROPE_DTYPE_BF16, fake, ts, tst, fake, ts, tst,
                                              ROPE_DTYPE_BF16, 7, sl, NULL),
           ROPE_ERR_INVALID, "mode");
    expect("odd slice length", rope_partial_fwd_inplace(fake, xs, ROPE_DTYPE_BF16, fake, ts, tst, fake, ts, tst,
                                                        ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, bad_sl, NULL),
           ROPE_ERR_INVALID, "even");
    expect("table of the wrong length", rope_partial_check(fake, xs, ROPE_DTYPE_F32, fake, xs, tst, fake, ts, tst,
                                                           ROPE_DTYPE_F32, ROPE_MODE_ROTATE_HALF, sl),
           ROPE_ERR_INVALID, "r1");
    expect("empty slice, NULL everything", rope_partial_fwd_inplace(NULL, xs, ROPE_DTYPE_F16, NULL, NULL, NULL,
                                                                    NULL, NULL, NULL, ROPE_DTYPE_F16,
                                                                    ROPE_MODE_INTERLEAVE, empty_sl, NULL),
           ROPE_OK, NULL);
    expect("empty tensor", rope_partial_bwd_out(NULL, NULL, xs_empty, ROPE_DTYPE_F32, NULL, NULL, NULL, NULL,
                                                NULL, NULL, ROPE_DTYPE_F32, ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_OK, NULL);
    expect("out of place, overlapping", rope_partial_fwd_out((char*)fake + 2, fake, xs, ROPE_DTYPE_BF16, fake, ts,
                                                             tst, fake, ts, tst, ROPE_DTYPE_BF16,
                                                             ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_INVALID, "overlap");
    expect("out of place, NULL y", rope_partial_bwd_out(NULL, fake, xs, ROPE_DTYPE_BF16, fake, ts, tst, fake, ts,
                                                        tst, ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_NULLPTR, "y is NULL");
    int64_t shapes[2][4] = {{2, 4, 3, 64}, {2, 5, 1, 64}};
    void* xs2[2] = {fake, fake_y};
    expect("multi, second tensor mismatched", rope_partial_fwd_inplace_multi(
               2, xs2, (const int64_t(*)[4])shapes, ROPE_DTYPE_BF16, fake, ts, tst, fake, ts, tst,
               ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_INVALID, "tensor 1");
    int64_t info[ROPE_LAUNCH_INFO_LEN];
    expect("launch plan", rope_partial_launch_info(fake, xs, ROPE_DTYPE_BF16, fake, ts, tst, fake, ts, tst,
                                                   ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, sl, info),
           ROPE_OK, NULL);
    if (info[0] != ROPE_KERNEL_VECTOR || info[2] <= 0) FAIL("launch plan: kernel %lld", (long long)info[0]);
    const int64_t* fake_pos = (const int64_t*)fake;
    const double* fake_f = (const double*)fake;
    int64_t ps[2] = {1, 4}, pst[2] = {4, 1}, ps_bad[2] = {3, 4};
    expect("positions NULL", rope_partial_fwd_inplace_pos(fake, xs, ROPE_DTYPE_BF16, NULL, ps, pst, fake_f,
                                                          ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_NULLPTR, "positions is NULL");
    expect("positions of 3 batches for 2", rope_partial_bwd_inplace_pos(fake, xs, ROPE_DTYPE_BF16, fake_pos, ps_bad,
                                                                        pst, fake_f, ROPE_DTYPE_BF16,
                                                                        ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_INVALID, "dimension B");
    expect("positions, empty slice, NULL everything", rope_partial_fwd_inplace_pos(
               NULL, xs, ROPE_DTYPE_F16, NULL, NULL, NULL, NULL, ROPE_DTYPE_F16, ROPE_MODE_ROTATE_HALF, empty_sl,
               NULL),
           ROPE_OK, NULL);
    expect("out of place positions, overlapping", rope_partial_fwd_out_pos(
               (char*)fake + 2, fake, xs, ROPE_DTYPE_BF16, fake_pos, ps, pst, fake_f, ROPE_DTYPE_BF16,
               ROPE_MODE_INTERLEAVE, sl, NULL),
           ROPE_ERR_INVALID, "overlap");
    expect("position launch plan", rope_partial_launch_info_pos(fake, xs, ROPE_DTYPE_BF16, fake_pos, ps, pst,
                                                                fake_f, ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, sl,
                                                                info),
           ROPE_OK, NULL);
    if (info[0] != ROPE_KERNEL_VECTOR || info[2] <= 0) FAIL("position launch plan: kernel %lld", (long long)info[0]);
}

int main(int argc, char** argv)
{
    g_state = 20261202u;
    check_errors();
    if (argc > 1 && strcmp(argv[1], "--no-gpu") == 0) {
        printf("all ok\n");
        return 0;
    }
    int ndev = 0;
    HIP_OK(hipGetDeviceCount(&ndev));
    if (ndev < 1) FAIL("no GPU");
    static const Case cases[] = {
        {"bf16 long-context-like, lanes [32,96), per-batch tables, fwd in place",
         {2, 64, 8, 128}, ROPE_DTYPE_BF16, ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, 0, {32, 96}, {2, 64, 1, 64}, 0, 0, 1},
        {"bf16 MLA-like, lanes [0,64) of 192, bwd in place",
         {1, 32, 16, 192}, ROPE_DTYPE_BF16, ROPE_DTYPE_BF16, ROPE_MODE_INTERLEAVE, 1, {0, 64}, {1, 32, 1, 64}, 0, 0, 0},
        {"fp32 rotate_half, bwd out of place",
         {1, 16, 4, 64}, ROPE_DTYPE_F32, ROPE_DTYPE_F32, ROPE_MODE_ROTATE_HALF, 1, {0, 64}, {1, 16, 1, 64}, 1, 0, 0},
        {"bf16 x with fp32 tables, fwd out of place",
         {2, 16, 6, 128}, ROPE_DTYPE_BF16, ROPE_DTYPE_F32, ROPE_MODE_INTERLEAVE, 0, {32, 96}, {2, 16, 1, 64}, 1, 0, 1},
        {"fp16 Q and K (8 and 2 heads) in one call, fwd",
         {2, 32, 8, 64}, ROPE_DTYPE_F16, ROPE_DTYPE_F16, ROPE_MODE_INTERLEAVE, 0, {0, 64}, {1, 32, 1, 64}, 2, 2, 1},
        {"fp16 odd start [3,35) (general kernel), bwd in place",
         {1, 8, 3, 40}, ROPE_DTYPE_F16, ROPE_DTYPE_F16, ROPE_MODE_INTERLEAVE, 1, {3, 35}, {1, 8, 1, 32}, 0, 0, 0},
        {"bf16 rotate_half with per-head tables, fwd in place",
         {2, 8, 4, 128}, ROPE_DTYPE_BF16, ROPE_DTYPE_BF16, ROPE_MODE_ROTATE_HALF, 0, {32, 96}, {2, 8, 4, 64}, 0, 0, 0},
    };
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) run_case(&cases[i]);
    const int64_t pxs[4] = {2, 64, 8, 128}, psl[2] = {32, 96}, pxs2[4] = {3, 16, 5, 64}, psl2[2] = {0, 64};
    run_pos_case("bf16 positions, lanes [32,96), bwd in place", pxs, ROPE_DTYPE_BF16, ROPE_DTYPE_BF16,
                 ROPE_MODE_INTERLEAVE, 1, psl, 500000.0);
    run_pos_case("fp32 positions, rotate_half, fwd in place", pxs2, ROPE_DTYPE_F32, ROPE_DTYPE_F32,
                 ROPE_MODE_ROTATE_HALF, 0, psl2, 10000.0);
    HIP_OK(hipGetLastError());
    printf("all ok\n");
    return 0;
}
