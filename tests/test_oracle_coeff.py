"""Pins of the oracle's rotary coefficient (mode value c >= 2).

"ascend-transformer-boost 的 MlaPreprocessOperation", section 2, gives the
rotation coefficients qRotaryCoeff / kRotaryCoeff: 2 for the half rotation,
4 or headDim also allowed. Read as: the slice splits into c parts of H = L/c
lanes, and lane k of part 2g pairs with lane k of part 2g+1, the even part
taking the negated partner. Pinned here against statements that do not share
the oracle's formula:

  C1 c = 2 is rotate_half and c = L is interleave, byte for byte
  C2 any c is rotate_half applied to each group of 2H lanes on its own
     (per-lane random tables, both directions)
  C3 the complex product on the pairs (2gH + k, 2gH + k + H) with one angle
     per pair
  C4 backward after forward is the identity on rotation tables (fp64 bound)
  C5 the tables from positions put pair i = gH + k at those two lanes
  C6 a coefficient that is odd or does not divide L is rejected
"""
import math

import numpy as np
import pytest

import oracle
from oracle_refs import assert_storage_equal, round_to, widen

DTYPES = ["f32", "f16", "bf16"]


def _x(shape, dtype, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return round_to(rng.standard_normal(shape) * scale, dtype)


def _run(x, shape, dtype, r1, r2, mode, sl, direction):
    y = np.array(x, copy=True)
    tdt = "f32" if r1.dtype == np.float32 else dtype
    oracle.rope_rows(y, shape, dtype, r1, r2, mode, sl, direction, table_dtype=tdt)
    return y


def _random_tables(shape4, dtype, seed):
    rng = np.random.default_rng(seed)
    return round_to(rng.standard_normal(shape4), dtype), round_to(rng.standard_normal(shape4), dtype)


def _pairs(L, c):
    """First and second lanes of the pairs, pair i = g*H + k in lane order."""
    H = L // c
    first = np.array([g * 2 * H + k for g in range(c // 2) for k in range(H)])
    return first, first + H


# ------------------------------------------------------------------ C1

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_c1_two_is_rotate_half_and_L_is_interleave(dtype, direction):
    shape, sl = (2, 3, 4, 48), (8, 40)
    L = sl[1] - sl[0]
    x = _x(shape, dtype, 1)
    r1, r2 = _random_tables((1, 3, 4, L), dtype, 2)
    assert_storage_equal(_run(x, shape, dtype, r1, r2, 2, sl, direction),
                         _run(x, shape, dtype, r1, r2, "rotate_half", sl, direction), dtype, "c = 2")
    assert_storage_equal(_run(x, shape, dtype, r1, r2, L, sl, direction),
                         _run(x, shape, dtype, r1, r2, "interleave", sl, direction), dtype, "c = L")


# ------------------------------------------------------------------ C2

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("L,c,start", [(32, 4, 0), (64, 4, 16), (48, 6, 2), (64, 8, 0), (24, 12, 4), (16, 16, 0)])
def test_c2_groups_rotate_half_independently(dtype, direction, L, c, start):
    D = start + L + 6
    shape = (2, 5, 3, D)
    sl = (start, start + L)
    x = _x(shape, dtype, L + c)
    r1, r2 = _random_tables((2, 5, 3, L), dtype, 3 * L + c)
    got = _run(x, shape, dtype, r1, r2, c, sl, direction)
    want = np.array(x, copy=True)
    G = 2 * (L // c)
    for g in range(c // 2):
        lo = start + g * G
        t1 = np.ascontiguousarray(r1[..., g * G:(g + 1) * G])
        t2 = np.ascontiguousarray(r2[..., g * G:(g + 1) * G])
        want = _run(want, shape, dtype, t1, t2, "rotate_half", (lo, lo + G), direction)
    assert_storage_equal(got, want, dtype, f"L={L} c={c}")


# ------------------------------------------------------------------ C3

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("L,c", [(32, 4), (64, 8), (40, 10), (64, 2), (64, 64)])
def test_c3_complex_product_on_the_pairs(dtype, L, c):
    shape = (1, 7, 2, L)
    sl = (0, L)
    rng = np.random.default_rng(L * 100 + c)
    x = _x(shape, dtype, L * 7 + c)
    theta = rng.uniform(-50, 50, size=(1, 7, 1, L // 2))
    first, second = _pairs(L, c)
    cos = np.empty((1, 7, 1, L))
    sin = np.empty((1, 7, 1, L))
    cos[..., first] = cos[..., second] = np.cos(theta)
    sin[..., first] = sin[..., second] = np.sin(theta)
    r1, r2 = round_to(cos, dtype), round_to(sin, dtype)
    got = _run(x, shape, dtype, r1, r2, c, sl, "fwd")
    xv = widen(x, dtype)
    cv, sv = widen(r1, dtype), widen(r2, dtype)
    z = (xv[..., first] + 1j * xv[..., second]) * (cv[..., first] + 1j * sv[..., first])
    want = np.array(xv, copy=True)
    want[..., first], want[..., second] = z.real, z.imag
    # both products are exact in fp64 (and in fp32 for 16-bit data), so each
    # side rounds the same exact sum: fp32 data once, 16-bit data through fp32
    assert_storage_equal(got, round_to(want, dtype), dtype, f"L={L} c={c}")


# ------------------------------------------------------------------ C4

@pytest.mark.parametrize("L,c", [(32, 4), (96, 6), (128, 8)])
def test_c4_backward_inverts_forward(L, c):
    shape = (2, 9, 3, L + 8)
    sl = (8, 8 + L)
    rng = np.random.default_rng(L + c)
    x = rng.standard_normal(shape).astype(np.float32)
    theta = rng.uniform(-1e4, 1e4, size=(1, 9, 1, L // 2))
    first, second = _pairs(L, c)
    cos = np.empty((1, 9, 1, L), np.float32)
    sin = np.empty((1, 9, 1, L), np.float32)
    cos[..., first] = cos[..., second] = np.cos(theta)
    sin[..., first] = sin[..., second] = np.sin(theta)
    y = _run(x, shape, "f32", cos, sin, c, sl, "fwd")
    back = _run(y, shape, "f32", cos, sin, c, sl, "bwd")
    # cos^2 + sin^2 = 1 within fp32 rounding of the tables; each step rounds to fp32
    assert np.max(np.abs(back.astype(np.float64) - x)) < 1e-5 * max(1.0, np.max(np.abs(x)))
    assert not np.array_equal(y, x)


# ------------------------------------------------------------------ C5

@pytest.mark.parametrize("L,c", [(16, 4), (24, 6), (32, 8)])
def test_c5_position_tables_place_pairs_by_part(L, c):
    pos = np.array([[0, 3, 70000], [5, 65535, 11]], dtype=np.int64)
    f = 500000.0 ** (-2.0 * np.arange(L // 2) / L)
    cs, sn = oracle.pos_tables(pos, f, L, c, "f32")
    H = L // c
    for b in range(2):
        for t in range(3):
            for i in range(L // 2):
                g, k = divmod(i, H)
                th = float(pos[b, t]) * float(f[i])
                for j in (2 * g * H + k, 2 * g * H + k + H):
                    assert cs[b, t, 0, j] == np.float32(math.cos(th)), (b, t, i, j)
                    assert sn[b, t, 0, j] == np.float32(math.sin(th)), (b, t, i, j)


# ------------------------------------------------------------------ C6

@pytest.mark.parametrize("c,L", [(3, 12), (6, 8), (16, 8), (5, 10), (-2, 8)])
def test_c6_undefined_coefficients_are_rejected(c, L):
    shape = (1, 2, 1, 16)
    x = _x(shape, "f32", 0)
    r = np.ones((1, 2, 1, L), np.float32)
    with pytest.raises(ValueError):
        oracle.rope_rows(np.array(x, copy=True), shape, "f32", r, r, c, (0, L), "fwd")
    with pytest.raises(ValueError):
        oracle.pos_tables(np.zeros((1, 2), np.int64), np.ones(L // 2), L, c, "f32")
