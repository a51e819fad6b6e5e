"""Pins for the CPU oracle of partial RoPE (the oracle against the mathematics).

Each test compares the oracle with a statement of the operation that does not
share its formula (see ``oracle_refs``), or with an invariant the mathematics
fixes:

  P1 interleave = complex multiplication of (x_2i + i·x_2i+1) by e^{iθ}
  P2 rotate_half = complex multiplication on the pairs (i, i+L/2), and a
     lane permutation of interleave
  P3 per-lane tables (random, not pair-duplicated) = the vector formula
  P4 backward = autograd gradient (Jacobian transpose); bwd∘fwd ≈ identity
  P5 rotation by a then by b ≈ rotation by a+b
  P6 per-pair norm preserved when cos²+sin²=1
  P7 position 0 (cos 1, sin 0) is an exact identity
  P8 empty slice / empty tensor are no-ops; lanes outside the slice untouched
  plus the broadcast layouts the constraints name, odd starts, special values.

Sources: "CANN ops-transformer 算子详解：inplace_partial_rotary_mul 原地部分旋转
位置编码" (sections 计算公式, 约束说明, 自动微分说明, and the mixed-precision
paragraph of the tiling/kernel section) and "ANE实战RoPE位置编码在MIL中的纯ANE
实现" (section 先搞懂RoPE and the backward section).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle_refs import (assert_storage_equal, backward_by_autograd, expand_tables,
                         rotate_complex_form, rotate_vector_form, round_to, widen)

DTYPES = ["f32", "f16", "bf16"]


def _rope_tables(x_shape, L, mode, dtype, tshape=None, base=10000.0, offsets=None):
    """Pair-structured cos/sin tables in storage form (independent of the
    workloads module, so that the tests also pin its recipe)."""
    B, S, N, _ = x_shape
    tshape = tshape or (1, S, 1, L)
    Bt = tshape[0]
    pos = np.arange(S, dtype=np.float64)[None, :] + (
        np.zeros((Bt, 1)) if offsets is None else np.asarray(offsets, np.float64)[:, None])
    i = np.arange(L // 2, dtype=np.float64)
    th = pos[:, :, None] * base ** (-2.0 * i / L)
    th = np.repeat(th, 2, axis=-1) if mode == "interleave" else np.concatenate([th, th], -1)
    c = round_to(np.cos(th).reshape(tshape), dtype)
    s = round_to(np.sin(th).reshape(tshape), dtype)
    return c, s


def _x(shape, dtype, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return round_to(rng.standard_normal(shape) * scale, dtype)


def _run(x, shape, dtype, r1, r2, mode, sl, direction, rows=None):
    y = np.array(x, copy=True)
    tdt = "f32" if r1.dtype == np.float32 else dtype
    oracle.rope_rows(y, shape, dtype, r1, r2, mode, sl, direction, rows=rows, table_dtype=tdt)
    return y


# ---------------------------------------------------------------- P1 / P2

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mode,shape,sl", [
    ("interleave", (2, 16, 3, 64), (0, 32)),
    ("interleave", (1, 8, 4, 128), (32, 96)),
    ("interleave", (1, 5, 2, 10), (3, 9)),          # odd start
    ("rotate_half", (2, 16, 3, 128), (0, 128)),
    ("rotate_half", (1, 8, 2, 192), (64, 192)),
    ("rotate_half", (1, 7, 2, 12), (1, 11)),        # odd start, L/2 odd
])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_matches_complex_rotation(dtype, mode, shape, sl, direction):
    L = sl[1] - sl[0]
    x = _x(shape, dtype, seed=zlib.crc32(repr((dtype, mode, sl)).encode()) % 1000)
    c, s = _rope_tables(shape, L, mode, dtype)
    got = _run(x, shape, dtype, c, s, mode, sl, direction)
    want = rotate_complex_form(widen(x, dtype), expand_tables(widen(c, dtype), shape, L),
                               expand_tables(widen(s, dtype), shape, L), sl[0], sl[1], mode,
                               inverse=(direction == "bwd"))
    assert_storage_equal(got, round_to(want, dtype), dtype, f"{mode} {direction}")


def test_counter_clockwise_quarter_turn():
    """θ = π/2 maps the pair (1, 0) to (0, 1): even lanes take the negated partner."""
    x = np.array([1.0, 0.0, 0.0, 1.0], np.float32).reshape(1, 1, 1, 4)
    c = np.zeros((1, 1, 1, 4), np.float32)
    s = np.ones((1, 1, 1, 4), np.float32)
    y = _run(x, x.shape, "f32", c, s, "interleave", (0, 4), "fwd")
    assert y.ravel().tolist() == [0.0, 1.0, -1.0, 0.0]
    y = _run(x, x.shape, "f32", c, s, "rotate_half", (0, 4), "fwd")
    # pairs (0,2) = (1,0) -> (0,1) and (1,3) = (0,1) -> (-1,0)
    assert y.ravel().tolist() == [0.0, -1.0, 1.0, 0.0]


@pytest.mark.parametrize("dtype", DTYPES)
def test_rotate_half_is_permuted_interleave(dtype):
    """rotate_half(x) = Pᵀ interleave(P x) with (Px)_2i = x_i, (Px)_2i+1 = x_i+L/2."""
    shape, sl = (2, 6, 3, 80), (8, 72)
    L, h = sl[1] - sl[0], (sl[1] - sl[0]) // 2
    rng = np.random.default_rng(5)
    x = round_to(rng.standard_normal(shape), dtype)
    c = round_to(rng.standard_normal((2, 6, 1, L)), dtype)
    s = round_to(rng.standard_normal((2, 6, 1, L)), dtype)
    perm = np.empty(L, np.int64)
    perm[0::2] = np.arange(h)
    perm[1::2] = np.arange(h) + h
    xp = x.copy()
    xp[..., sl[0]:sl[1]] = x[..., sl[0]:sl[1]][..., perm]
    for direction in ("fwd", "bwd"):
        a = _run(x, shape, dtype, c, s, "rotate_half", sl, direction)
        bperm = _run(xp, shape, dtype, np.ascontiguousarray(c[..., perm]),
                     np.ascontiguousarray(s[..., perm]), "interleave", sl, direction)
        b = bperm.copy()
        b[..., sl[0]:sl[1]][..., perm] = bperm[..., sl[0]:sl[1]]
        assert_storage_equal(a, b, dtype, direction)


# ---------------------------------------------------------------- P3 / P4

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_per_lane_tables_match_vector_formula(dtype, mode):
    """Random tables: sin multiplies the swapped value at the same lane."""
    shape, sl = (2, 8, 4, 96), (16, 80)
    L = sl[1] - sl[0]
    rng = np.random.default_rng(7)
    x = round_to(rng.standard_normal(shape), dtype)
    c = round_to(rng.standard_normal((2, 8, 1, L)), dtype)
    s = round_to(rng.standard_normal((2, 8, 1, L)), dtype)
    got = _run(x, shape, dtype, c, s, mode, sl, "fwd")
    want = rotate_vector_form(widen(x, dtype), expand_tables(widen(c, dtype), shape, L),
                              expand_tables(widen(s, dtype), shape, L), sl[0], sl[1], mode)
    assert_storage_equal(got, round_to(want, dtype), dtype, mode)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_backward_is_gradient(dtype, mode):
    """Backward = autograd gradient of the forward w.r.t. x (random tables,
    so the transpose differs from rotating by -θ)."""
    shape, sl = (2, 4, 3, 64), (8, 48)
    L = sl[1] - sl[0]
    rng = np.random.default_rng(8)
    g = round_to(rng.standard_normal(shape), dtype)
    c = round_to(rng.standard_normal((1, 4, 3, L)), dtype)
    s = round_to(rng.standard_normal((1, 4, 3, L)), dtype)
    got = _run(g, shape, dtype, c, s, mode, sl, "bwd")
    want = backward_by_autograd(widen(g, dtype), expand_tables(widen(c, dtype), shape, L),
                                expand_tables(widen(s, dtype), shape, L), sl[0], sl[1], mode)
    assert_storage_equal(got, round_to(want, dtype), dtype, mode)


@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_backward_is_dense_jacobian_transpose(mode):
    """Brute force on a tiny row: build J column by column from the forward,
    then dx = Jᵀ g."""
    shape, sl = (1, 1, 1, 8), (2, 8)
    L = sl[1] - sl[0]
    rng = np.random.default_rng(9)
    c = rng.standard_normal((1, 1, 1, L)).astype(np.float32)
    s = rng.standard_normal((1, 1, 1, L)).astype(np.float32)
    J = np.zeros((8, 8))
    for k in range(8):
        e = np.zeros(shape, np.float32)
        e.ravel()[k] = 1.0
        J[:, k] = widen(_run(e, shape, "f32", c, s, mode, sl, "fwd"), "f32").ravel()
    g = rng.standard_normal(shape).astype(np.float32)
    got = widen(_run(g, shape, "f32", c, s, mode, sl, "bwd"), "f32").ravel()
    np.testing.assert_allclose(got, J.T @ g.ravel().astype(np.float64), rtol=1e-6, atol=1e-7)
    # J is a 2x2 rotation-like block on each pair, identity outside the slice
    assert np.allclose(J[:2, :2], np.eye(2)) and np.allclose(J[:2, 2:], 0)


@pytest.mark.parametrize("dtype,tol_ulps", [("f32", 4), ("f16", 2), ("bf16", 2)])
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_bwd_after_fwd_is_identity(dtype, tol_ulps, mode):
    shape, sl = (2, 32, 2, 64), (0, 64)
    x = _x(shape, dtype, 10)
    c, s = _rope_tables(shape, 64, mode, "f32")
    if dtype != "f32":
        c, s = _rope_tables(shape, 64, mode, dtype)
    y = _run(x, shape, dtype, c, s, mode, sl, "fwd")
    z = _run(y, shape, dtype, c, s, mode, sl, "bwd")
    xv, zv = widen(x, dtype), widen(z, dtype)
    eps = {"f32": 2.0**-23, "f16": 2.0**-10, "bf16": 2.0**-7}[dtype]
    # tables rounded to 16 bits are not exactly unit, so allow their error too
    unit_err = 0 if dtype == "f32" else 2 * eps
    bound = tol_ulps * eps * np.abs(xv).max() + unit_err * np.abs(xv)
    assert np.all(np.abs(zv - xv) <= bound + 1e-30)


# ---------------------------------------------------------------- P5 / P6 / P7

def test_composition_of_rotations():
    shape, L = (1, 64, 2, 64), 64
    rng = np.random.default_rng(11)
    x = rng.standard_normal(shape).astype(np.float32)
    a = rng.uniform(-np.pi, np.pi, (1, 64, 1, L // 2))
    b = rng.uniform(-np.pi, np.pi, (1, 64, 1, L // 2))

    def tables(th):
        th = np.repeat(th, 2, axis=-1)
        return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)

    ca, sa = tables(a)
    cb, sb = tables(b)
    cab, sab = tables(a + b)
    y = _run(_run(x, shape, "f32", ca, sa, "interleave", (0, L), "fwd"), shape, "f32", cb, sb,
             "interleave", (0, L), "fwd")
    z = _run(x, shape, "f32", cab, sab, "interleave", (0, L), "fwd")
    np.testing.assert_allclose(y, z, rtol=0, atol=2e-6 * np.abs(x).max())


@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_pair_norm_preserved(mode):
    shape, sl = (2, 128, 4, 128), (0, 128)
    x = _x(shape, "f32", 12)
    c, s = _rope_tables(shape, 128, mode, "f32")
    y = _run(x, shape, "f32", c, s, mode, sl, "fwd").astype(np.float64)
    x = x.astype(np.float64)
    if mode == "interleave":
        nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    else:
        nx = x[..., :64] ** 2 + x[..., 64:] ** 2
        ny = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=2e-6, atol=1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_position_zero_is_identity(dtype, mode, direction):
    shape, sl = (1, 4, 3, 64), (0, 64)
    x = _x(shape, dtype, 13)
    c, s = _rope_tables(shape, 64, mode, dtype)
    y = _run(x, shape, dtype, c, s, mode, sl, direction)
    assert widen(c, dtype)[0, 0].min() == 1.0 and widen(s, dtype)[0, 0].max() == 0.0
    xv = widen(x, dtype)
    nz = xv[:, 0] != 0
    assert np.array_equal(np.asarray(y)[:, 0][nz], np.asarray(x)[:, 0][nz])
    assert np.array_equal(widen(y, dtype)[:, 0], xv[:, 0])  # zeros: equal by value


# ---------------------------------------------------------------- P8 and layouts

@pytest.mark.parametrize("dtype", DTYPES)
def test_noops_leave_buffer_identical(dtype):
    shape = (1, 16, 2, 64)
    x = _x(shape, dtype, 14)
    c, s = _rope_tables(shape, 32, "interleave", dtype)
    for sl in [(8, 8), (0, 0), None, (64, 64)]:
        for direction in ("fwd", "bwd"):
            y = _run(x, shape, dtype, c, s, "interleave", sl, direction)
            assert y.tobytes() == x.tobytes()
    empty = np.zeros((0, 16, 2, 64), x.dtype)
    y = _run(empty, (0, 16, 2, 64), dtype, c, s, "interleave", (0, 32), "fwd")
    assert y.size == 0


@pytest.mark.parametrize("dtype", DTYPES)
def test_lanes_outside_slice_untouched(dtype):
    shape, sl = (2, 8, 4, 128), (32, 96)
    x = _x(shape, dtype, 15)
    c, s = _rope_tables(shape, 64, "interleave", dtype, tshape=(2, 8, 1, 64), offsets=[5, 900])
    y = _run(x, shape, dtype, c, s, "interleave", sl, "fwd")
    assert y[..., :32].tobytes() == x[..., :32].tobytes()
    assert y[..., 96:].tobytes() == x[..., 96:].tobytes()
    assert not np.array_equal(y[..., 32:96], x[..., 32:96])


@pytest.mark.parametrize("tshape", [(2, 8, 4, 32), (2, 1, 4, 32), (2, 1, 1, 32),
                                    (1, 1, 1, 32), (2, 8, 1, 32), (1, 8, 1, 32), (1, 8, 4, 32)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_broadcast_layouts(tshape, dtype):
    """BSND, B1ND, B11D, 111D, BS1D tables (and more), random values: the
    oracle reads the broadcast index, pinned against explicit expansion."""
    shape, sl = (2, 8, 4, 48), (6, 38)
    rng = np.random.default_rng(16)
    x = round_to(rng.standard_normal(shape), dtype)
    c = round_to(rng.standard_normal(tshape), dtype)
    s = round_to(rng.standard_normal(tshape), dtype)
    for direction in ("fwd", "bwd"):
        got = _run(x, shape, dtype, c, s, "interleave", sl, direction)
        ce, se = expand_tables(widen(c, dtype), shape, 32), expand_tables(widen(s, dtype), shape, 32)
        if direction == "fwd":
            want = rotate_vector_form(widen(x, dtype), ce, se, sl[0], sl[1], "interleave")
        else:
            want = backward_by_autograd(widen(x, dtype), ce, se, sl[0], sl[1], "interleave")
        assert_storage_equal(got, round_to(want, dtype), dtype, f"{tshape} {direction}")
    # a zero-stride view (numpy broadcast_to) reads the same values
    cb = np.broadcast_to(c, (2, 8, 4, 32))
    sb = np.broadcast_to(s, (2, 8, 4, 32))
    got2 = _run(x, shape, dtype, cb, sb, "interleave", sl, "fwd")
    want2 = _run(x, shape, dtype, c, s, "interleave", sl, "fwd")
    assert got2.tobytes() == want2.tobytes()


@pytest.mark.parametrize("dtype", DTYPES)
def test_row_subset_equals_full_tensor(dtype):
    shape, sl = (3, 10, 4, 64), (16, 48)
    x = _x(shape, dtype, 17)
    c, s = _rope_tables(shape, 32, "interleave", dtype, tshape=(3, 10, 1, 32), offsets=[0, 7, 99])
    full = _run(x, shape, dtype, c, s, "interleave", sl, "bwd")
    rows = np.array([0, 5, 17, 63, 119], np.int64)
    sub = np.ascontiguousarray(x.reshape(-1, 64)[rows])
    oracle.rope_rows(sub, shape, dtype, c, s, "interleave", sl, "bwd", rows=rows)
    assert sub.tobytes() == full.reshape(-1, 64)[rows].tobytes()


@pytest.mark.parametrize("dtype", DTYPES)
def test_special_values(dtype):
    """NaN propagates, infinities follow IEEE products, overflow rounds to inf."""
    big = {"f32": 3e38, "f16": 60000.0, "bf16": 3e38}[dtype]
    vals = np.array([np.nan, 1.0, np.inf, 1.0, big, big, -big, big, 0.0, -0.0], np.float64)
    x = round_to(vals, dtype).reshape(1, 1, 1, 10)
    c = round_to(np.ones(10), dtype).reshape(1, 1, 1, 10)
    s = round_to(np.full(10, 0.5), dtype).reshape(1, 1, 1, 10)
    got = _run(x, x.shape, dtype, c, s, "interleave", (0, 10), "fwd")
    want = rotate_vector_form(widen(x, dtype), widen(c, dtype), widen(s, dtype), 0, 10, "interleave")
    assert_storage_equal(got, round_to(want, dtype), dtype)
    g = widen(got, dtype).ravel()
    assert np.isnan(g[0]) and np.isnan(g[1])        # NaN partner spreads to the pair
    assert np.isinf(g[5])                           # big + big/2 overflows to +inf


def test_rejects_undefined_arguments():
    x = np.zeros((1, 1, 1, 8), np.float32)
    c = np.zeros((1, 1, 1, 3), np.float32)
    for sl in [(0, 3), (-1, 3), (4, 2), (0, 10)]:
        with pytest.raises(ValueError):
            oracle.rope_rows(x, x.shape, "f32", c, c, "interleave", sl, "fwd")


def test_workload_tables_follow_recipe():
    """The shared input generator builds the tables these pins assume."""
    for name in ("c0", "c1", "c2", "c3"):
        w = W.WORKLOADS[name]
        r1, r2 = W.make_tables(w)
        c, s = _rope_tables(w.x_shapes[0], w.L, w.mode, w.dtype, tshape=w.table_shape)
        assert W.to_numpy_storage(r1).tobytes() == c.tobytes(), name
        assert W.to_numpy_storage(r2).tobytes() == s.tobytes(), name


# ---------------------------------------------------------------- mixed precision

def _exact_rotation(xv, cv, sv, sl, mode, direction):
    """fp64 rotation of widened values (exact products), for error bounds."""
    L = sl[1] - sl[0]
    if direction == "fwd":
        return rotate_vector_form(xv, cv, sv, sl[0], sl[1], mode)
    return backward_by_autograd(xv, cv, sv, sl[0], sl[1], mode)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_mixed_fp32_tables_within_one_ulp_of_exact(dtype, mode, direction):
    """16-bit x with fp32 tables: the fp32 product and sum roundings stay
    below one ulp of the 16-bit result, so the oracle is within 1 ulp of the
    exact rotation rounded to the storage type."""
    shape, sl = (2, 8, 4, 96), (16, 80)
    L = sl[1] - sl[0]
    rng = np.random.default_rng(21)
    x = round_to(rng.standard_normal(shape), dtype)
    th = rng.uniform(-np.pi, np.pi, (2, 8, 1, L))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    got = _run(x, shape, dtype, c, s, mode, sl, direction)
    exact = _exact_rotation(widen(x, dtype), expand_tables(c.astype(np.float64), shape, L),
                            expand_tables(s.astype(np.float64), shape, L), sl, mode, direction)
    want = round_to(exact, dtype)
    g = got.view(np.int16).astype(np.int64)
    w = want.view(np.int16).astype(np.int64)
    ordered = lambda i: np.where(i < 0, -32768 - i, i)
    assert np.abs(ordered(g) - ordered(w)).max() <= 1


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mixed_tables_holding_16_bit_values_match_16_bit_tables(dtype):
    """fp32 tables whose values are 16-bit numbers give the 16-bit-table
    result bit for bit (both products are then exact)."""
    shape, sl = (2, 8, 4, 64), (0, 64)
    rng = np.random.default_rng(22)
    x = round_to(rng.standard_normal(shape), dtype)
    c16 = round_to(rng.standard_normal((2, 8, 1, 64)), dtype)
    s16 = round_to(rng.standard_normal((2, 8, 1, 64)), dtype)
    c32, s32 = widen(c16, dtype).astype(np.float32), widen(s16, dtype).astype(np.float32)
    for mode in ("interleave", "rotate_half"):
        for direction in ("fwd", "bwd"):
            a = _run(x, shape, dtype, c16, s16, mode, sl, direction)
            b = np.array(x, copy=True)
            oracle.rope_rows(b, shape, dtype, c32, s32, mode, sl, direction, table_dtype="f32")
            assert a.tobytes() == b.tobytes()
